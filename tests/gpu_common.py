"""Helpers of the GPU tests: device contexts for the synthetic workloads and
the oracle's reference values (live for small inputs, stored for large ones)."""
from __future__ import annotations

import json
import os

import numpy as np

from synth import make_instance, make_weights, workload

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_weights_cache = {}


def host_weights(idx):
    if idx not in _weights_cache:
        _weights_cache.clear()      # keep at most one large model in host memory
        _weights_cache[idx] = make_weights(workload(idx))
    return _weights_cache[idx]


def device_context(idx, n_pages, max_pos, max_tok, weights_dev=None):
    from shared_prefix_kv_amd import jev
    wl = workload(idx)
    m = wl.model
    if weights_dev is None:
        weights_dev = jev.upload_weights(host_weights(idx))
    desc = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps,
                         max_pos, max_tok)
    return jev.Context(desc, n_pages, weights_dev), weights_dev


def golden(idx):
    """Stored oracle probabilities; the fingerprint must match today's inputs."""
    from tests.golden.make_golden import fingerprint
    path = os.path.join(GOLD, f"probs_w{idx}.json")
    with open(path) as f:
        g = json.load(f)
    wl = workload(idx)
    fp = fingerprint(wl, make_instance(wl), host_weights(idx))
    assert g["fingerprint"] == fp, "stored oracle values were made from different inputs"
    return g


def split_probs(probs_dev, loff):
    p = probs_dev.float().cpu().numpy()
    return [p[loff[i]:loff[i + 1]] for i in range(len(loff) - 1)]


def max_abs(a_list, b_list):
    return max(float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) for a, b in zip(a_list, b_list))


def row_rel_err(got, ref):
    """Per (token, head) row: ||a - b|| / max(||b||, 1e-6); returns the max."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    num = np.linalg.norm(g - r, axis=-1)
    den = np.maximum(np.linalg.norm(r, axis=-1), 1e-6)
    return float(np.max(num / den))


# ------------------------------------------------------------------ parity report
# Every parity check records its worst error and its bar here before it
# asserts; the terminal summary (tests/conftest.py) prints the table, so a
# quiet run still shows the numbers.
PARITY_LOG = []


def record(what, err, bar):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0].split("::")[-1]
    PARITY_LOG.append((test, what, float(err), float(bar)))
    print(f"{what}: {err:.3e} (bar {bar:.1e})", flush=True)


def stored_bars(g, pass_index=0):
    """Per-branch bars of a stored workload: max(1e-3, 3 * spread), the spread
    being how far the oracle's own probabilities move under other accumulation
    orders (tests/golden/make_golden.py)."""
    from tests.golden.make_golden import bars
    ps = g["passes"][pass_index]
    assert "spread" in ps and ps.get("by_order"), "stored oracle values carry no spread"
    return bars(ps["spread"])


def check_branches(what, got, ref, bars):
    """Asserts |got_b - ref_b|_inf <= bars[b] for every branch b; records the
    worst error, the worst error relative to its bar and that bar."""
    errs = [float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) for a, b in zip(got, ref)]
    assert len(errs) == len(bars) and len(errs) > 0
    worst = max(range(len(errs)), key=lambda i: errs[i] / bars[i])
    record(f"{what} (worst branch {worst}, max err {max(errs):.2e})", errs[worst], bars[worst])
    bad = [(i, e, b) for i, (e, b) in enumerate(zip(errs, bars)) if e > b]
    assert not bad, f"{what}: branches over their bars (branch, err, bar): {bad[:8]}"
    return errs
