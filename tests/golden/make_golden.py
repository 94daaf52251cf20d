"""Writes the oracle's label probabilities for the large workloads, and the
per-branch accumulation-order spread that the bf16 parity bars derive from.

    python -m tests.golden.make_golden [--orders fp64,fp32_krev,fp32_khalves] 2 3 4 5 6

Calls only ``oracle`` (and ``synth`` for the seeded inputs).  Each listed
branch is recomputed from scratch by the oracle (no prefix sharing) with
float32 accumulation; the output files ``probs_w<index>.json`` hold the
probabilities with a fingerprint of the inputs so that a change of the
generator is caught instead of silently comparing against stale values.

Spread.  The same branches are recomputed with alternative arithmetic of
``oracle.model``: float64 products and sums; float32 with the contraction
index reversed; float32 over two halves of the contraction; float32 for the
steps between contractions (RMSNorm, RoPE, softmax, residual add) as well.
Every one is a faithful implementation of the same definition, so how far
they move a branch's probabilities is the floor below which no
implementation with another rounding order can be held: a bf16 rounding that
one order lands on one side of, another lands on the other, and random-weight
bf16 models carry such flips through their blocks.  ``spread`` is, per branch, the largest
absolute change over the alternatives; the parity tests hold branch b to
max(1e-3, 3 * spread[b]).  Orders already stored are kept when the
fingerprint matches, so alternatives can be added one run at a time.

Workload 5 is scored on a seeded subset of branches per pass (first, last and
two drawn ones) because one from-scratch branch of 32,896 tokens costs about
93 TFLOP on the CPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import time

import numpy as np

from oracle import model as om
from synth import make_instance, make_weights, workload

HERE = os.path.dirname(os.path.abspath(__file__))
# alternative -> (accumulation of the contractions, precision between them)
ALTERNATIVES = {"fp64": ("fp64", "fp64"), "fp32_krev": ("fp32_krev", "fp64"),
                "fp32_khalves": ("fp32_khalves", "fp64"), "ew32": ("fp32", "fp32")}
ALT_ORDERS = tuple(ALTERNATIVES)
BAR_FLOOR = 1e-3
BAR_FACTOR = 3.0


def fingerprint(wl, inst, weights) -> str:
    h = hashlib.sha256()
    for p in range(len(inst.passes) or 1):
        for s, lab in inst.full_sequences(p):
            h.update(np.asarray(s, np.int32).tobytes())
            h.update(np.asarray(lab, np.int32).tobytes())
    for a in (weights.embed[:3], weights.unembed[-3:], weights.wq[0][:2], weights.wo[-1][-2:]):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def subset(wl, n_branches: int, pass_index: int):
    if wl.index != 5:
        return list(range(n_branches))
    rng = np.random.default_rng([wl.index, 3, pass_index])
    extra = sorted(int(x) for x in rng.choice(np.arange(1, n_branches - 1), size=2, replace=False))
    return sorted({0, n_branches - 1, *extra})


def bars(spread):
    """Per-branch bars from the stored spread (the rule the parity tests use)."""
    return [max(BAR_FLOOR, BAR_FACTOR * s) for s in spread]


def _score(m, seqs, sel, tag, idx, p):
    out = []
    for b in sel:
        t1 = time.time()
        pr = om.score_from_scratch(m, [seqs[b][0]], [seqs[b][1]])[0]
        out.append([float(x) for x in pr])
        print(f"w{idx} {tag} pass {p} branch {b}: {time.time() - t1:.1f}s", flush=True)
    return out


def main(indices, orders):
    for idx in indices:
        wl = workload(idx)
        t0 = time.time()
        w = make_weights(wl)
        inst = make_instance(wl)
        fp = fingerprint(wl, inst, w)
        path = os.path.join(HERE, f"probs_w{idx}.json")
        old = None
        if os.path.exists(path):
            with open(path) as f:
                old = json.load(f)
            if old.get("fingerprint") != fp:
                old = None
        out = {"workload": wl.name, "index": wl.index, "fingerprint": fp,
               "produced_by": "oracle.model.score_from_scratch (from-scratch, no prefix sharing)",
               "bar_rule": f"per branch max({BAR_FLOOR}, {BAR_FACTOR} * spread)",
               "passes": []}
        n_pass = len(inst.passes) if wl.kind != "tree" else 1
        m32 = None
        for p in range(n_pass):
            seqs = inst.full_sequences(p)
            sel = subset(wl, len(seqs), p)
            prev = old["passes"][p] if old else {}
            if prev.get("branches") == sel:
                probs = prev["probs"]
            else:
                m32 = m32 or om.from_weights(w)
                probs = _score(m32, seqs, sel, "fp32", idx, p)
            by_order = dict(prev.get("by_order", {})) if prev.get("branches") == sel else {}
            out["passes"].append({"branches": sel, "probs": probs, "by_order": by_order})
        for order in orders:
            if all(order in ps["by_order"] for ps in out["passes"]):
                continue
            gemm, ew = ALTERNATIVES[order]
            m_alt = om.from_weights(w, gemm=gemm, elementwise=ew)
            for p, ps in enumerate(out["passes"]):
                if order not in ps["by_order"]:
                    ps["by_order"][order] = _score(m_alt, inst.full_sequences(p), ps["branches"],
                                                   order, idx, p)
            del m_alt
        for ps in out["passes"]:
            ref = np.asarray(ps["probs"])
            ps["spread"] = [float(max((np.max(np.abs(np.asarray(alt[i]) - ref[i]))
                                       for alt in ps["by_order"].values()), default=0.0))
                            for i in range(len(ref))]
        out["orders"] = sorted({o for ps in out["passes"] for o in ps["by_order"]})
        out["oracle_seconds"] = round(time.time() - t0 + (old or {}).get("oracle_seconds", 0.0), 1)
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
        for ps in out["passes"]:
            print(f"w{idx} spread", ["%.2e" % s for s in ps["spread"]], flush=True)
        print("wrote", path, flush=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("indices", nargs="*", type=int, default=[2, 3, 4, 5, 6])
    ap.add_argument("--orders", default=",".join(ALT_ORDERS))
    a = ap.parse_args()
    main(a.indices, [o for o in a.orders.split(",") if o])
