"""Token-prefix tree, staged submission rounds and KV page assignment.

Test infrastructure only (see the package docstring).  An independent Python
statement of the planner that the host library implements in C++; the two
must agree bit for bit.

Source: LLM2Jev shared-prefix page.  Its "why is the same material computed
several times" section describes candidates that share a state, then a
question's instructions, then differ in one criterion; its staged-submission
section builds a shared prefix first and submits the candidates that reuse it
in later rounds, with independent branches sharing a round and the number of
rounds following the token tree; its Radix Cache section says reuse is keyed
on the exact token prefix and that each candidate's last scored position is
always computed.  Page size 16 tokens.

Readings (the pages leave these open):

* Trie: compressed, token-granular, over each candidate's tokens after its
  resident match.  A node is a maximal token run shared by the same set of
  candidates.
* Dissolution: top-down, a node that has children, where no candidate ends,
  and whose own run is shorter than one page, is removed; its tokens are
  prepended to each child.  Short accidental common runs therefore never add a
  round.
* Rounds, mode "depth": level-synchronous by depth under the anchor (round k
  computes every new node at depth k).
* Rounds, mode "candidate_first" (the staged-submission section's own
  example order): a candidate is submitted in a round when the first node on
  its path that is not yet computed either has no children (nothing there for
  others to reuse) or is a shared node of which it is the smallest candidate
  (it builds that prefix for the others).  A submitted candidate computes
  every node of its path not yet computed; a candidate is scored in the round
  its read-out node is computed.  Nodes of a round are in (depth, smallest
  candidate) order.
* Canonical order: (depth, smallest candidate index through the node); node
  ids are ranks in that order.
* Pages: free ids in a min-heap; each new node takes ceil(len/16) lowest ids at
  its round, in canonical order; every node starts on a fresh page.  Nodes
  without children are released when their round ends, the plan's internal
  nodes when the call ends.
* Resident match: walk resident nodes from the root, taking the longest child
  segment that matches in full and still leaves at least one token (the last
  scored position must be computed).
* Reuse inside a resident node (a scoring or planning call over full
  candidates): where no child continues in full, the child sharing the
  longest run rounded down to whole pages (at least one page, leaving at
  least one token; ties to the earliest created) is split at that page
  boundary, and the candidate continues the first part.  The split keeps the
  original handle, references and children on the second part.  Candidates are
  resolved in input order, each on the tree the earlier ones left.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

PAGE = 16


def n_pages_for(n_tokens: int) -> int:
    return (n_tokens + PAGE - 1) // PAGE


class PoolExhausted(Exception):
    pass


class PagePool:
    def __init__(self, n_pages: int):
        self.n_pages = n_pages
        self.free = list(range(n_pages))
        heapq.heapify(self.free)

    def alloc(self, n: int) -> List[int]:
        if n > len(self.free):
            raise PoolExhausted(n)
        return [heapq.heappop(self.free) for _ in range(n)]

    def release(self, pages: Sequence[int]) -> None:
        for p in pages:
            heapq.heappush(self.free, p)

    def take(self, pages: Sequence[int]) -> None:
        """Marks the given free ids as used."""
        gone = set(pages)
        if not gone <= set(self.free):
            raise ValueError("page not free")
        self.free = [p for p in self.free if p not in gone]
        heapq.heapify(self.free)

    def n_free(self) -> int:
        return len(self.free)


@dataclass
class ResNode:
    handle: int
    parent: int            # 0 = empty root
    tokens: Tuple[int, ...]
    pages: List[int]
    start: int             # logical position of the first token
    refs: int = 1
    children: List[int] = field(default_factory=list)   # handles, creation order
    last_use: int = 0     # stamp of the last call that used the node


class ResidentTree:
    """Resident prefixes, each owning its pages; handles are creation serials."""

    def __init__(self, pool: PagePool):
        self.pool = pool
        self.nodes: Dict[int, ResNode] = {}
        self.root_children: List[int] = []
        self.next_handle = 1
        self.keep = False      # cache policy: keep prefixes whose last reference is dropped
        self.evictions = 0

    def _children(self, parent: int) -> List[int]:
        return self.root_children if parent == 0 else self.nodes[parent].children

    def end_pos(self, h: int) -> int:
        if h == 0:
            return 0
        n = self.nodes[h]
        return n.start + len(n.tokens)

    def path_pages(self, h: int) -> List[Tuple[int, int]]:
        """(page id, valid tokens) of every page on the path root..h."""
        chain = []
        while h != 0:
            chain.append(self.nodes[h])
            h = self.nodes[h].parent
        out = []
        for n in reversed(chain):
            L = len(n.tokens)
            for i, p in enumerate(n.pages):
                out.append((p, min(PAGE, L - PAGE * i)))
        return out

    def prefill(self, items: Sequence[Tuple[int, Sequence[int]]]) -> List[int]:
        """Creates (or re-references) one node per (parent, tokens), in order.

        All-or-nothing: raises PoolExhausted before any change if the new
        nodes do not fit.  An existing child with the identical segment is
        re-used (one more reference, no pages)."""
        need, seen = 0, set()
        for parent, toks in items:
            if parent != 0 and parent not in self.nodes:
                raise KeyError(parent)
            key = (parent, tuple(int(t) for t in toks))
            if self._find_child(parent, key[1]) is None and key not in seen:
                seen.add(key)
                need += n_pages_for(len(toks))
        if need > self.pool.n_free():
            raise PoolExhausted(need)
        out = []
        for parent, toks in items:
            toks = tuple(int(t) for t in toks)
            h = self._find_child(parent, toks)
            if h is not None:
                self.nodes[h].refs += 1
                out.append(h)
                continue
            h = self.next_handle
            self.next_handle += 1
            self.nodes[h] = ResNode(h, parent, toks, self.pool.alloc(n_pages_for(len(toks))),
                                    self.end_pos(parent))
            self._children(parent).append(h)
            out.append(h)
        return out

    def _find_child(self, parent: int, toks: Tuple[int, ...]) -> Optional[int]:
        for c in self._children(parent):
            if self.nodes[c].tokens == toks:
                return c
        return None

    def adopt(self, parent: int, toks: Sequence[int], pages: Sequence[int]) -> int:
        """A new node continuing `parent` whose K/V are already in `pages`
        (free ids, taken here); one reference."""
        self.pool.take(pages)
        h = self.next_handle
        self.next_handle += 1
        self.nodes[h] = ResNode(h, parent, tuple(int(t) for t in toks), list(pages), self.end_pos(parent))
        self._children(parent).append(h)
        return h

    def release(self, h: int) -> None:
        """Drops one caller reference; without the cache policy, frees nodes
        left with no reference and no child."""
        n = self.nodes[h]
        n.refs -= 1
        if self.keep:
            return
        while n is not None and n.refs == 0 and not n.children:
            self.pool.release(n.pages)
            del self.nodes[n.handle]
            sib = self._children(n.parent)
            sib.remove(n.handle)
            n = self.nodes.get(n.parent)

    # ---- cache policy (openjev-multimodal performance page, repeated-state
    # section: a state's KV is kept for the next request that repeats it, and
    # several states can be kept and used in turn).  Reading: a cached prefix
    # (no caller reference) without resident children may be evicted when a
    # call is short of pages, least recently used first, ties to the smallest
    # handle, never one on the path of a prefix the call uses.

    def path(self, h: int) -> List[int]:
        out = []
        while h != 0:
            out.append(h)
            h = self.nodes[h].parent
        return out

    def stamp(self, handles: Sequence[int], t: int) -> None:
        for h in handles:
            for x in self.path(h):
                self.nodes[x].last_use = t

    def victim(self, pinned: set) -> Optional[int]:
        cands = [n for n in self.nodes.values() if n.refs == 0 and not n.children and n.handle not in pinned]
        if not cands:
            return None
        return min(cands, key=lambda n: (n.last_use, n.handle)).handle

    def evict(self, h: int) -> None:
        n = self.nodes.pop(h)
        self.pool.release(n.pages)
        self._children(n.parent).remove(h)
        self.evictions += 1

    def split(self, h: int, at: int) -> int:
        """First `at` tokens (whole pages) of node h become a new node in its
        place; h keeps the rest below it.  Returns the new handle."""
        tail = self.nodes[h]
        nh = self.next_handle
        self.next_handle += 1
        head = ResNode(nh, tail.parent, tail.tokens[:at], tail.pages[:at // PAGE], tail.start, refs=0,
                       children=[h], last_use=tail.last_use)
        sib = self._children(tail.parent)
        sib[sib.index(h)] = nh
        tail.parent = nh
        tail.tokens = tail.tokens[at:]
        tail.pages = tail.pages[at // PAGE:]
        tail.start += at
        self.nodes[nh] = head
        return nh

    def match_split(self, seq: Sequence[int]) -> Tuple[int, int]:
        """match(), then page-aligned reuse inside the child that shares the
        longest whole-page run below it (splitting that child)."""
        h, pos = self.match(seq)
        rest = [int(t) for t in seq[pos:len(seq) - 1]]     # the last token is always computed
        choice, reuse = None, 0
        for c in self._children(h):
            t = self.nodes[c].tokens
            common = 0
            for a, b in zip(t, rest):
                if a != b:
                    break
                common += 1
            pages = common // PAGE * PAGE
            if PAGE <= pages < len(t) and pages > reuse:
                choice, reuse = c, pages
        if choice is None:
            return h, pos
        return self.split(choice, reuse), pos + reuse

    def match(self, seq: Sequence[int]) -> Tuple[int, int]:
        """Deepest resident node whose whole path is a prefix of seq with at
        least one token of seq left over; returns (handle, matched length)."""
        h, pos = 0, 0
        seq = [int(t) for t in seq]
        while True:
            best = None
            for c in self._children(h):
                t = self.nodes[c].tokens
                if pos + len(t) < len(seq) and tuple(seq[pos:pos + len(t)]) == t:
                    if best is None or len(t) > len(self.nodes[best].tokens):
                        best = c
            if best is None:
                return h, pos
            h, pos = best, pos + len(self.nodes[best].tokens)


@dataclass
class PlanNode:
    cands: List[int]          # candidate indices through this node (sorted)
    a: int                    # segment [a, b) relative to the anchor
    b: int
    anchor: int
    readout: List[int] = field(default_factory=list)
    children: List["PlanNode"] = field(default_factory=list)
    parent: Optional["PlanNode"] = None
    depth: int = 0
    node_id: int = -1
    pages: List[int] = field(default_factory=list)

    @property
    def cand_min(self) -> int:
        return self.cands[0]


def _build(cands: List[int], a: int, rel: Dict[int, List[int]], anchor: int) -> List[PlanNode]:
    groups: Dict[int, List[int]] = {}
    order: List[int] = []
    for c in cands:
        if len(rel[c]) == a:
            continue
        t = rel[c][a]
        if t not in groups:
            groups[t] = []
            order.append(t)
        groups[t].append(c)
    out = []
    for t in order:
        part = groups[t]
        b = a + 1
        while all(len(rel[c]) > b for c in part) and len({rel[c][b] for c in part}) == 1:
            b += 1
        node = PlanNode(part, a, b, anchor, readout=[c for c in part if len(rel[c]) == b])
        node.children = _build([c for c in part if len(rel[c]) > b], b, rel, anchor)
        out.append(node)
    return out


def _dissolve(nodes: List[PlanNode]) -> List[PlanNode]:
    out: List[PlanNode] = []
    queue = list(nodes)
    while queue:
        n = queue.pop(0)
        if n.children and not n.readout and (n.b - n.a) < PAGE:
            for ch in n.children:
                ch.a = n.a
            queue = n.children + queue
            continue
        out.append(n)
    out.sort(key=lambda x: x.cand_min)
    for n in out:
        n.children = _dissolve(n.children)
    return out


@dataclass
class Plan:
    rounds: List[List[PlanNode]]
    anchors: List[int]            # per candidate: resident handle it continues
    anchor_len: List[int]         # per candidate: tokens matched in the resident tree
    readout_node: List[int]       # per candidate: node id it is read out at
    released_after_round: List[List[int]]

    def serialize(self) -> List[int]:
        """Flat int32 image compared bit for bit with the host library."""
        out = [len(self.rounds)]
        for rnd in self.rounds:
            out.append(len(rnd))
            for n in rnd:
                out += [n.node_id, n.parent.node_id if n.parent else -1, n.anchor, n.depth,
                        n.cand_min, n.a, n.b - n.a, len(n.pages)] + n.pages
                out += [len(n.readout)] + n.readout
        out.append(len(self.readout_node))
        for c in range(len(self.readout_node)):
            out += [self.anchors[c], self.anchor_len[c], self.readout_node[c]]
        return out


def _paths(tops: List[PlanNode]) -> Dict[int, List[PlanNode]]:
    """Candidate -> its nodes from the top-level node down to its read-out node."""
    out: Dict[int, List[PlanNode]] = {}

    def walk(node: PlanNode, above: List[PlanNode]) -> None:
        here = above + [node]
        for c in node.readout:
            out[c] = here
        for ch in node.children:
            walk(ch, here)

    for t in tops:
        walk(t, [])
    return out


def _rounds_candidate_first(tops: List[PlanNode]) -> List[List[PlanNode]]:
    paths = _paths(tops)
    computed: set = set()
    pending = sorted(paths)
    rounds: List[List[PlanNode]] = []
    while pending:
        submitted = []
        for c in pending:
            first = next(x for x in paths[c] if id(x) not in computed)
            if not first.children or first.cand_min == c:
                submitted.append(c)
        new: Dict[int, PlanNode] = {}
        for c in submitted:
            for x in paths[c]:
                if id(x) not in computed:
                    new[id(x)] = x
        computed |= set(new)
        rounds.append(sorted(new.values(), key=lambda x: (x.depth, x.cand_min)))
        pending = [c for c in pending if id(paths[c][-1]) not in computed]
    return rounds


def plan_candidates(tree: ResidentTree, seqs: Sequence[Sequence[int]], mode: str = "depth") -> Plan:
    """Plans the staged rounds of a call and assigns pages (all-or-nothing).

    Pages of nodes without children are returned to the pool at the end of
    their round, the rest at the end of the plan (i.e. this function leaves
    the pool as it found it once the plan has run; the caller replays that
    with ``release_plan``)."""
    n = len(seqs)
    anchors, alen, rel = [], [], {}
    for c, s in enumerate(seqs):
        h, m = tree.match(s)
        anchors.append(h)
        alen.append(m)
        rel[c] = [int(t) for t in s[m:]]
    by_anchor: Dict[int, List[int]] = {}
    for c in range(n):
        by_anchor.setdefault(anchors[c], []).append(c)
    tops: List[PlanNode] = []
    for h, cs in by_anchor.items():
        tops += _dissolve(_build(cs, 0, rel, h))
    # depth levels (and parents)
    levels: List[List[PlanNode]] = []
    frontier = sorted(tops, key=lambda x: x.cand_min)
    d = 1
    while frontier:
        for x in frontier:
            x.depth = d
        levels.append(sorted(frontier, key=lambda x: x.cand_min))
        nxt = []
        for x in frontier:
            for ch in x.children:
                ch.parent = x
                nxt.append(ch)
        frontier = nxt
        d += 1
    if mode == "candidate_first":
        levels = _rounds_candidate_first(tops)
    elif mode != "depth":
        raise ValueError(mode)
    nid = 0
    for lvl in levels:
        for x in lvl:
            x.node_id = nid
            nid += 1
    # page assignment with a dry run first (all-or-nothing)
    free_snapshot = list(tree.pool.free)
    released: List[List[int]] = []
    try:
        for lvl in levels:
            for x in lvl:
                x.pages = tree.pool.alloc(n_pages_for(x.b - x.a))
            rel_ids = [x.node_id for x in lvl if not x.children]
            for x in lvl:
                if not x.children:
                    tree.pool.release(x.pages)
            released.append(rel_ids)
        for lvl in levels:
            for x in lvl:
                if x.children:
                    tree.pool.release(x.pages)
    except PoolExhausted:
        tree.pool.free = free_snapshot
        raise
    readout_node = [-1] * n
    for lvl in levels:
        for x in lvl:
            for c in x.readout:
                readout_node[c] = x.node_id
    return Plan(levels, anchors, alen, readout_node, released)


def plan_with_reuse(tree: ResidentTree, seqs: Sequence[Sequence[int]], mode: str = "depth") -> Plan:
    """The plan of a scoring call, on a copy of the tree: anchors resolved with
    reuse inside resident nodes (splits), then plan_candidates.  The given
    tree and its pool are left unchanged."""
    import copy
    t = copy.deepcopy(tree)
    for s in seqs:
        t.match_split(s)
    return plan_candidates(t, seqs, mode)


def branch_pages(tree: ResidentTree, parents: Sequence[int],
                 suffixes: Sequence[Sequence[int]]) -> List[List[int]]:
    """Pages of one explicit scoring call: each branch is a new leaf under its
    parent, allocated in input order and released when the call ends."""
    need = sum(n_pages_for(len(s)) for s in suffixes)
    if need > tree.pool.n_free():
        raise PoolExhausted(need)
    out = [tree.pool.alloc(n_pages_for(len(s))) for s in suffixes]
    for p in out:
        tree.pool.release(p)
    return out


class Session:
    """Call-level model of the host library's resident state: the tree, the
    cache policy, the plan mode and one recency stamp per call."""

    def __init__(self, n_pages: int, mode: str = "depth", keep: bool = False):
        self.tree = ResidentTree(PagePool(n_pages))
        self.tree.keep = keep
        self.mode = mode
        self.clock = 0

    def _copy(self) -> "ResidentTree":
        import copy
        return copy.deepcopy(self.tree)

    def _room(self, pinned: set, fits) -> None:
        """Evicts cached prefixes (found on a copy first) until fits(tree)."""
        if fits(self.tree):
            return
        if not self.tree.keep:
            raise PoolExhausted(0)
        t = self._copy()
        victims = []
        while not fits(t):
            v = t.victim(pinned)
            if v is None:
                raise PoolExhausted(0)
            t.evict(v)
            victims.append(v)
        for v in victims:
            self.tree.evict(v)

    def _pins(self, handles: Sequence[int]) -> set:
        return {x for h in handles for x in self.tree.path(h)}

    def prefill(self, items: Sequence[Tuple[int, Sequence[int]]]) -> List[int]:
        used = []
        for parent, toks in items:
            used.append(parent)
            c = self.tree._find_child(parent, tuple(int(t) for t in toks))
            if c is not None:
                used.append(c)

        def fits(t: ResidentTree) -> bool:
            need, seen = 0, set()
            for parent, toks in items:
                key = (parent, tuple(int(x) for x in toks))
                if t._find_child(parent, key[1]) is None and key not in seen:
                    seen.add(key)
                    need += n_pages_for(len(toks))
            return need <= t.pool.n_free()

        self._room(self._pins(used), fits)
        out = self.tree.prefill(items)
        self.clock += 1
        self.tree.stamp(out, self.clock)
        return out

    def release(self, handles: Sequence[int]) -> None:
        self.clock += 1
        for h in handles:
            self.tree.stamp([h], self.clock)
            self.tree.release(h)

    def _plan_pins(self, tree: ResidentTree, seqs) -> set:
        return {x for s in seqs for x in tree.path(tree.match(s)[0])}

    def plan(self, seqs) -> Plan:
        """The plan scoring would run now, splits and evictions included;
        changes nothing."""
        t = self._copy()
        for s in seqs:
            t.match_split(s)
        pins = self._plan_pins(t, seqs)
        while True:
            try:
                return plan_candidates(t, seqs, self.mode)
            except PoolExhausted:
                v = t.victim(pins) if t.keep else None
                if v is None:
                    raise
                t.evict(v)

    def set_keep(self, keep: bool) -> None:
        self.tree.keep = keep
        if not keep:
            while True:
                v = self.tree.victim(set())
                if v is None:
                    break
                self.tree.evict(v)

    def stats(self) -> Dict[str, int]:
        nodes = self.tree.nodes.values()
        return {"pages_in_use": self.tree.pool.n_pages - self.tree.pool.n_free(),
                "resident_prefixes": len(self.tree.nodes),
                "cached_prefixes": sum(1 for n in nodes if n.refs == 0),
                "cached_pages": sum(len(n.pages) for n in nodes if n.refs == 0),
                "evictions": self.tree.evictions}


class Scheduler:
    """Round-level continuous batching of requests on one session (the shared-
    prefix scoring article's "next steps" name cross-request continuous
    batching for throughput; this is the reading built here).

    A request is a list of candidates.  Each step: the requests submitted since
    the last step join the active ones; the unfinished candidates of all active
    requests (request order, then candidate order) are planned together like
    one scoring call (reuse inside resident nodes, depth rounds, evictions
    under the cache policy), and only the first round runs.  Its nodes with
    children become resident nodes held by the scheduler, so that the next
    step continues below them; candidates read out in that round are done.
    Held nodes that no unfinished candidate of a started request passes
    through (by its resident match) are then released, oldest first; a
    request still waiting pins nothing, since it might never fit beside what
    it would pin.  Every step therefore advances each
    active request by one level of its candidate tree, and new requests join
    at their first level in the same GPU round.

    Admission: a request that does not fit an empty pool on its own is
    refused at submission.  When a step's plan does not fit, the newest
    request that has not taken part in a step yet is left out of it (it waits
    for a later step), until the plan fits; if the started requests alone do
    not fit, the step fails and changes nothing."""

    def __init__(self, session: Session):
        self.s = session
        self.queued: List[Tuple[int, List[List[int]]]] = []
        self.active: List[dict] = []
        self.done_tickets: List[int] = []
        self.held: List[int] = []
        self.next_ticket = 1

    def submit(self, seqs: Sequence[Sequence[int]]) -> int:
        alone = ResidentTree(PagePool(self.s.tree.pool.n_pages))
        plan_candidates(alone, seqs, "depth")            # raises PoolExhausted
        t = self.next_ticket
        self.next_ticket += 1
        self.queued.append((t, [[int(x) for x in q] for q in seqs]))
        return t

    def status(self, ticket: int) -> int:
        """0 queued, 1 active, 2 finished."""
        if any(t == ticket for t, _ in self.queued):
            return 0
        if any(r["ticket"] == ticket for r in self.active):
            return 1
        if ticket in self.done_tickets:
            return 2
        raise KeyError(ticket)

    def _stage(self, seqs):
        """A scoring call's tree work on a copy: splits in candidate order, the
        plan, evictions under the cache policy (none in the candidates' paths)."""
        import copy
        t = copy.deepcopy(self.s.tree)
        for q in seqs:
            t.match_split(q)
        pins = {x for q in seqs for x in t.path(t.match(q)[0])}
        while True:
            try:
                return t, plan_candidates(t, seqs, "depth")
            except PoolExhausted:
                v = t.victim(pins) if t.keep else None
                if v is None:
                    raise
                t.evict(v)

    def step(self) -> Optional[Plan]:
        """Runs one round; returns the plan it was taken from (None if idle)."""
        import copy
        for t, seqs in self.queued:
            self.active.append({"ticket": t, "seqs": seqs, "done": [False] * len(seqs), "started": False})
        self.queued = []
        incl = [True] * len(self.active)
        while True:
            cands = [(ri, ci) for ri, r in enumerate(self.active) if incl[ri] for ci in range(len(r["seqs"]))
                     if not r["done"][ci]]
            if not cands:
                return None
            seqs = [self.active[ri]["seqs"][ci] for ri, ci in cands]
            try:
                t, plan = self._stage(seqs)
                break
            except PoolExhausted:
                later = [ri for ri in range(len(self.active)) if incl[ri] and not self.active[ri]["started"]]
                if not later:
                    raise
                incl[later[-1]] = False
        for ri in range(len(self.active)):
            if incl[ri]:
                self.active[ri]["started"] = True
        self.s.tree = t
        self.s.clock += 1
        t.stamp(plan.anchors, self.s.clock)
        made = []
        for x in plan.rounds[0]:
            if x.children:
                c0 = x.cand_min
                off = plan.anchor_len[c0]
                made.append(t.adopt(x.anchor, seqs[c0][off + x.a:off + x.b], x.pages))
        t.stamp(made, self.s.clock)
        self.held += made
        for x in plan.rounds[0]:
            for c in x.readout:
                ri, ci = cands[c]
                self.active[ri]["done"][ci] = True
        still = []
        for r in self.active:
            if all(r["done"]):
                self.done_tickets.append(r["ticket"])
            else:
                still.append(r)
        self.active = still
        needed = set()
        for r in self.active:
            for ci, q in enumerate(r["seqs"]):
                if r["started"] and not r["done"][ci]:
                    needed |= set(t.path(t.match(q)[0]))
        keep_held = []
        for h in self.held:
            if h in needed:
                keep_held.append(h)
            else:
                t.release(h)
        self.held = keep_held
        return plan
