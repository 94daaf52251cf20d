"""Writes the oracle's label probabilities for the large workloads.

    python -m tests.golden.make_golden 2 3 4 5

Calls only ``oracle`` (and ``synth`` for the seeded inputs).  Each listed
branch is recomputed from scratch by the oracle (no prefix sharing); the
output files ``probs_w<index>.json`` hold the probabilities with a fingerprint
of the inputs so that a change of the generator is caught instead of silently
comparing against stale values.  Workload 5 is scored on a seeded subset of
branches per pass (first, last and two drawn ones) because one from-scratch
branch of 32,896 tokens costs about 93 TFLOP on the CPU.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

from oracle import model as om
from synth import make_instance, make_weights, workload

HERE = os.path.dirname(os.path.abspath(__file__))


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


def main(indices):
    for idx in indices:
        wl = workload(idx)
        t0 = time.time()
        w = make_weights(wl)
        inst = make_instance(wl)
        m = om.from_weights(w)
        out = {"workload": wl.name, "index": wl.index, "fingerprint": fingerprint(wl, inst, w),
               "produced_by": "oracle.model.score_from_scratch (from-scratch, no prefix sharing)",
               "passes": []}
        n_pass = len(inst.passes) if wl.kind != "tree" else 1
        for p in range(n_pass):
            seqs = inst.full_sequences(p)
            sel = subset(wl, len(seqs), p)
            probs = []
            for b in sel:
                t1 = time.time()
                pr = om.score_from_scratch(m, [seqs[b][0]], [seqs[b][1]])[0]
                probs.append([float(x) for x in pr])
                print(f"w{idx} pass {p} branch {b}: {time.time() - t1:.1f}s", flush=True)
            out["passes"].append({"branches": sel, "probs": probs})
        out["oracle_seconds"] = round(time.time() - t0, 1)
        path = os.path.join(HERE, f"probs_w{idx}.json")
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
        print("wrote", path, flush=True)


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [2, 3, 4, 5])
