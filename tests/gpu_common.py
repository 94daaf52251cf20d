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
