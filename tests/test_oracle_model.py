"""Pins of the oracle's forward pass against closed forms, invariants, a
library routine and a pure-Python brute force (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle.bf16 import bits_to_f32, round_bf16
from synth import ModelShape, Request, Workload, make_weights
from tests import brute


def tiny_workload(index=101, **kw):
    shape = dict(n_layers=2, d=8, hq=4, hkv=2, dh=4, vocab=11, dtype="f32")
    shape.update(kw)
    return Workload(index, "tiny", ModelShape(**shape),
                    requests=(Request(prefix_len=4, n_branches=1, suffix_len=2, k_labels=2),))


def f64_model(wl, std=None):
    w = make_weights(wl)
    if std is not None:  # larger weights make the attention pattern non-trivial
        for name in ("embed", "unembed"):
            setattr(w, name, getattr(w, name) * (std / 0.02))
        for lst in (w.wq, w.wk, w.wv, w.wo):
            for i in range(len(lst)):
                lst[i] = lst[i] * (std / 0.02)
    return om.from_weights(w, mode="f64"), w


# ---------------------------------------------------------------- bf16
def test_bf16_matches_torch_conversion():
    x = np.random.default_rng(3).standard_normal(200000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(round_bf16(x), ref)


def test_bf16_ties_to_even_and_f64_direct():
    one = 1.0
    assert round_bf16(np.float64(one + 2 ** -8)) == 1.0            # tie -> even (down)
    assert round_bf16(np.float64(one + 3 * 2 ** -8)) == one + 2 ** -6  # tie -> even (up)
    assert round_bf16(np.float64(one + 2 ** -8 + 2 ** -40)) == one + 2 ** -7  # above tie
    bits = np.array([0x3F80, 0xBF00, 0x4049], np.uint16)
    assert list(bits_to_f32(bits)) == [1.0, -0.5, np.float32(3.140625)]


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])
    y = om.rmsnorm(x, np.array([1.0, 2.0]), 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [[3 / r, 8 / r]], rtol=0, atol=1e-15)
    c = np.full((1, 16), -2.5)
    y = om.rmsnorm(c, np.ones(16), 1e-6)
    assert np.allclose(y, -2.5 / math.sqrt(6.25 + 1e-6), rtol=0, atol=1e-15)


def test_rmsnorm_scale_invariance():
    x = np.random.default_rng(1).standard_normal((5, 64))
    assert np.allclose(om.rmsnorm(x, np.ones(64), 0.0), om.rmsnorm(37.0 * x, np.ones(64), 0.0),
                       rtol=0, atol=1e-13)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_identity_and_norm():
    x = np.random.default_rng(2).standard_normal((3, 2, 8))
    assert np.allclose(om.rope(x, np.zeros(3, np.int64), 1e4), x, rtol=0, atol=0)
    y = om.rope(x, np.array([5, 77, 32000]), 1e4)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)


def test_rope_rotate_half_pairing():
    # dh = 4: pairs (0,2) and (1,3); frequency of pair 0 is 1 rad per position.
    x = np.zeros((1, 1, 4))
    x[0, 0, 0] = 1.0
    y = om.rope(x, np.array([1]), 1e4)[0, 0]
    assert np.allclose(y, [math.cos(1), 0, math.sin(1), 0], atol=1e-15)
    x = np.zeros((1, 1, 4))
    x[0, 0, 1] = 1.0
    f = 1e4 ** -0.5
    y = om.rope(x, np.array([3]), 1e4)[0, 0]
    assert np.allclose(y, [0, math.cos(3 * f), 0, math.sin(3 * f)], atol=1e-15)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    for (t, u, c) in [(7, 3, 100), (0, 0, 31999), (50, 49, 12345)]:
        a = (om.rope(q, np.array([t]), 1e4) * om.rope(k, np.array([u]), 1e4)).sum()
        b = (om.rope(q, np.array([t + c]), 1e4) * om.rope(k, np.array([u + c]), 1e4)).sum()
        assert abs(a - b) < 1e-10


# ---------------------------------------------------------------- attention
def _m64(hq=2, hkv=1, dh=4):
    wl = tiny_workload(hq=hq, hkv=hkv, dh=dh)
    return om.from_weights(make_weights(wl), mode="f64")


def test_attention_single_key_returns_v():
    m = _m64()
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((1, 2, 4)), rng.standard_normal((1, 1, 4)), rng.standard_normal((1, 1, 4))
    out = om.attention(m, q, k, v, np.array([0]), np.array([0]))
    assert np.allclose(out[0, 0], v[0, 0]) and np.allclose(out[0, 1], v[0, 0])


def test_attention_zero_query_is_causal_mean():
    m = _m64()
    rng = np.random.default_rng(6)
    n = 6
    q = np.zeros((n, 2, 4))
    k, v = rng.standard_normal((n, 1, 4)), rng.standard_normal((n, 1, 4))
    out = om.attention(m, q, k, v, np.arange(n), np.arange(n))
    for t in range(n):
        assert np.allclose(out[t, 1], v[: t + 1, 0].mean(axis=0), atol=1e-14)


def test_attention_matches_brute_force_and_torch_sdpa():
    m = _m64(hq=4, hkv=2, dh=8)
    rng = np.random.default_rng(7)
    n = 9
    q = rng.standard_normal((n, 4, 8)) * 2
    k = rng.standard_normal((n, 2, 8)) * 2
    v = rng.standard_normal((n, 2, 8))
    out = om.attention(m, q, k, v, np.arange(n), np.arange(n))
    # brute force, pure Python
    for t in range(n):
        for j in range(4):
            g = j // 2
            sc = [sum(q[t, j, e] * k[u, g, e] for e in range(8)) / math.sqrt(8) for u in range(t + 1)]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            ref = [sum(w[u] * v[u, g, e] for u in range(t + 1)) / sum(w) for e in range(8)]
            assert np.allclose(out[t, j], ref, atol=1e-13)
    # library routine (CPU, float64), KV heads expanded by the group mapping j // G
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(np.repeat(k, 2, axis=1)).permute(1, 0, 2)
    tv = torch.from_numpy(np.repeat(v, 2, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_attention_gqa_mapping_is_floor_division():
    m = _m64(hq=4, hkv=2, dh=4)
    rng = np.random.default_rng(8)
    n = 5
    q = rng.standard_normal((n, 4, 4))
    k, v = rng.standard_normal((n, 2, 4)), rng.standard_normal((n, 2, 4))
    out = om.attention(m, q, k, v, np.arange(n), np.arange(n))
    for j in range(4):
        single = om.attention(m, q[:, j:j + 1], k[:, j // 2:j // 2 + 1], v[:, j // 2:j // 2 + 1],
                              np.arange(n), np.arange(n))
        assert np.allclose(out[:, j], single[:, 0], atol=1e-15)
    # the other plausible mapping (j mod Hkv) must differ on this input
    assert not np.allclose(out[:, 1], om.attention(m, q[:, 1:2], k[:, 1:2], v[:, 1:2],
                                                   np.arange(n), np.arange(n))[:, 0])


def test_lse_merge_identity():
    """Softmax attention over a key set split in two equals the log-sum-exp
    merge of the two partial results (the identity the branch kernel uses)."""
    rng = np.random.default_rng(9)
    s = rng.standard_normal(40) * 3
    v = rng.standard_normal((40, 6))

    def part(idx):
        m = s[idx].max()
        w = np.exp(s[idx] - m)
        return (w[:, None] * v[idx]).sum(0) / w.sum(), m + math.log(w.sum())

    full, _ = part(np.arange(40))
    (o1, l1), (o2, l2) = part(np.arange(0, 17)), part(np.arange(17, 40))
    mx = max(l1, l2)
    merged = (math.exp(l1 - mx) * o1 + math.exp(l2 - mx) * o2) / (math.exp(l1 - mx) + math.exp(l2 - mx))
    assert np.allclose(merged, full, atol=1e-14)


# ---------------------------------------------------------------- whole model
def _lists(a):
    return np.asarray(a, np.float64).tolist()


def test_whole_model_matches_pure_python_brute_force():
    wl = tiny_workload(index=102)
    m, w = f64_model(wl, std=0.5)
    tokens = [3, 7, 0, 10, 3, 5]
    layers = [dict(g=_lists(m.attn_norm[l]), wq=_lists(m.wq[l]), wk=_lists(m.wk[l]),
                   wv=_lists(m.wv[l]), wo=_lists(m.wo[l])) for l in range(m.n_layers)]
    ref = brute.forward_last(tokens, _lists(m.embed), _lists(m.unembed), layers,
                             _lists(m.final_norm), m.hq, m.hkv, m.dh, m.theta, m.eps)
    got = om.full_logprobs(m, om.final_hidden(m, tokens))
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_shared_prefix_equals_from_scratch_f64():
    wl = tiny_workload(index=103, d=32, hq=4, hkv=2, dh=8, vocab=50)
    m, _ = f64_model(wl, std=0.3)
    rng = np.random.default_rng(10)
    prefix = rng.integers(0, 50, 20)
    cache = om.prefill_cache(m, prefix)
    for _ in range(3):
        suf = rng.integers(0, 50, int(rng.integers(1, 6)))
        a = om.final_hidden_with_cache(m, cache, len(prefix), suf)
        b = om.final_hidden(m, np.concatenate([prefix, suf]))
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_label_probs_from_logits_equal_from_logprobs():
    wl = tiny_workload(index=104, vocab=40)
    m, _ = f64_model(wl, std=0.5)
    h = om.final_hidden(m, [1, 2, 3])
    lp = om.full_logprobs(m, h)
    z = m.unembed @ h
    lab = [5, 17, 3]
    assert np.allclose(om.label_softmax(lp[lab]), om.label_softmax(z[lab]), atol=1e-15)


def test_bf16_mode_rounds_at_storage_points():
    """bf16 mode: the final hidden state is a bf16 value, and the bf16-mode
    result stays close to the float64 result (drift of storage rounding)."""
    wl = tiny_workload(index=105, dtype="bf16", d=64, hq=4, hkv=2, dh=16, vocab=97)
    w = make_weights(wl)
    mb = om.from_weights(w)
    mf = om.from_weights(w, mode="f64")
    assert mb.mode == "bf16"
    toks = [1, 50, 3, 96, 7, 7, 2]
    hb = om.final_hidden(mb, toks)
    assert np.array_equal(round_bf16(hb), hb)
    hf = om.final_hidden(mf, toks)
    assert np.max(np.abs(hb - hf)) < 0.05 * np.max(np.abs(hf))


# ---------------------------------------------------------------- bf16 storage points
def _bf16_pin_model(index=106):
    """Tiny bf16 model, float64 products and sums (so that the only roundings
    are the storage points), weights scaled by 16 (a power of two keeps them
    bf16 values) to make every storage rounding change the result."""
    wl = tiny_workload(index=index, dtype="bf16", d=16, hq=4, hkv=2, dh=8, vocab=23)
    m = om.from_weights(make_weights(wl), gemm="fp64")
    assert m.mode == "bf16" and m.gemm_dtype == np.float64
    m.embed *= 16.0
    m.unembed *= 16.0
    for lst in (m.wq, m.wk, m.wv, m.wo):
        for a in lst:
            a *= 16.0
    return m


def _brute_bf16(m, tokens, round_at):
    layers = [dict(g=_lists(m.attn_norm[l]), wq=_lists(m.wq[l]), wk=_lists(m.wk[l]),
                   wv=_lists(m.wv[l]), wo=_lists(m.wo[l])) for l in range(m.n_layers)]
    return np.asarray(brute.forward_last(tokens, _lists(m.embed), _lists(m.unembed), layers,
                                         _lists(m.final_norm), m.hq, m.hkv, m.dh, m.theta, m.eps,
                                         round_at=round_at))


BF16_TOKENS = [3, 7, 0, 22, 3, 5, 19]


def test_brute_bf16_rounding_is_ieee_round_to_nearest_even():
    x = np.random.default_rng(12).standard_normal(5000).astype(np.float32) * 5
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(np.array([brute.bf16(float(v)) for v in x], np.float32), ref)
    assert brute.bf16(1.0 + 2 ** -8) == 1.0 and brute.bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
    assert brute.bf16(255.5) == 256.0 and brute.bf16(-1.0 - 2 ** -7 - 2 ** -30) == -1.0 - 2 ** -7


def test_bf16_mode_matches_brute_force_storage_points():
    """The oracle's bf16 mode rounds exactly at the reading's storage points:
    RMSNorm outputs, q and k after RoPE, v, the attention output, the residual
    stream after each add, the final norm output (and nowhere else)."""
    m = _bf16_pin_model()
    got = om.full_logprobs(m, om.final_hidden(m, BF16_TOKENS))
    ref = _brute_bf16(m, BF16_TOKENS, brute.STORE_POINTS)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("change", ["drop:" + p for p in brute.STORE_POINTS] + ["qk_before_rope"])
def test_bf16_pin_tells_every_storage_point_apart(change):
    """Each storage point left out, or q/k rounded before RoPE instead of
    after, moves the brute-force result far beyond the pin's 1e-12: the pin
    above would catch that mistake in the oracle."""
    m = _bf16_pin_model()
    got = om.full_logprobs(m, om.final_hidden(m, BF16_TOKENS))
    if change == "qk_before_rope":
        pts = [p for p in brute.STORE_POINTS if p != "qk"] + ["qk_before_rope"]
    else:
        pts = [p for p in brute.STORE_POINTS if p != change.split(":")[1]]
    assert np.max(np.abs(got - _brute_bf16(m, BF16_TOKENS, pts))) > 1e-7


@pytest.mark.parametrize("order", om.GEMM_ORDERS)
def test_contractions_within_the_float_error_bound(order):
    """Every accumulation of ``contract`` is the exact product within the
    classical bound |err| <= gamma_k * sum |a_i b_i|, gamma_k = k u / (1 - k u),
    with u the unit roundoff of its precision (2^-24 float32, 2^-53 float64)."""
    wl = tiny_workload(index=107)
    m = om.from_weights(make_weights(wl), gemm=order)
    rng = np.random.default_rng(13)
    a = rng.standard_normal((7, 300)).astype(np.float32)
    b = rng.standard_normal((300, 9)).astype(np.float32)
    exact = a.astype(np.float64) @ b.astype(np.float64)
    got = np.asarray(om.contract(m, a, b), np.float64)
    u = 2.0 ** -53 if order == "fp64" else 2.0 ** -24
    k = a.shape[1]
    gamma = k * u / (1 - k * u)
    bound = gamma * (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64))
    assert np.all(np.abs(got - exact) <= bound)
    if order != "fp64":
        assert np.max(np.abs(got - exact)) > 0      # it really is a float32 accumulation


def test_attention_query_chunks_and_skipped_keys():
    """Queries processed in chunks of 3 with the keys a chunk cannot see skipped
    give the unchunked result and the pure-Python definition; the case is a
    suffix over cached keys (queries at positions 6..16, keys 0..16)."""
    m = _m64(hq=4, hkv=2, dh=8)
    rng = np.random.default_rng(14)
    nk, nq = 17, 11
    k = rng.standard_normal((nk, 2, 8)) * 2
    v = rng.standard_normal((nk, 2, 8))
    q = rng.standard_normal((nq, 4, 8)) * 2
    qp, kp = np.arange(nk - nq, nk), np.arange(nk)
    full = om.attention(m, q, k, v, qp, kp)
    chunked = om.attention(m, q, k, v, qp, kp, q_chunk=3)
    assert np.allclose(chunked, full, rtol=0, atol=1e-13)
    for t in range(nq):
        for j in range(4):
            g = j // 2
            vis = [u for u in range(nk) if kp[u] <= qp[t]]
            sc = [sum(q[t, j, e] * k[u, g, e] for e in range(8)) / math.sqrt(8) for u in vis]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            ref = [sum(w[i] * v[u, g, e] for i, u in enumerate(vis)) / sum(w) for e in range(8)]
            assert np.allclose(chunked[t, j], ref, rtol=0, atol=1e-13)


def test_attention_threaded_heads_match_single_head_calls():
    """Above 65,536 query-key pairs the heads run on a thread pool; each head
    equals the same head computed alone."""
    m = _m64(hq=4, hkv=2, dh=4)
    rng = np.random.default_rng(15)
    n = 260
    q = rng.standard_normal((n, 4, 4))
    k, v = rng.standard_normal((n, 2, 4)), rng.standard_normal((n, 2, 4))
    out = om.attention(m, q, k, v, np.arange(n), np.arange(n))
    for j in range(4):
        single = om.attention(m, q[:, j:j + 1], k[:, j // 2:j // 2 + 1], v[:, j // 2:j // 2 + 1],
                              np.arange(n), np.arange(n))
        assert np.array_equal(out[:, j], single[:, 0])


def test_float32_elementwise_steps_within_their_precision():
    """The float32 variants of RMSNorm, RoPE and the attention softmax (used
    only to measure the spread of faithful implementations) agree with the
    float64 closed forms to float32 precision, and really are float32."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((6, 64))
    g = rng.standard_normal(64)
    y32 = om.rmsnorm(x.astype(np.float32), g, 1e-6, np.float32)
    assert y32.dtype == np.float32
    y64 = om.rmsnorm(x.astype(np.float32), g, 1e-6)
    assert np.max(np.abs(y32 - y64) / np.maximum(np.abs(y64), 1e-3)) < 1e-5
    assert np.max(np.abs(y32 - y64)) > 0
    q = rng.standard_normal((5, 2, 16)).astype(np.float32)
    r32 = om.rope(q, np.array([0, 3, 100, 4000, 32000]), 1e4, np.float32)
    r64 = om.rope(q, np.array([0, 3, 100, 4000, 32000]), 1e4)
    assert r32.dtype == np.float32 and np.max(np.abs(r32 - r64)) < 1e-5
    w = make_weights(tiny_workload(index=108, dtype="bf16", d=16, hq=4, hkv=2, dh=8, vocab=23))
    m32 = om.from_weights(w, elementwise="fp32")
    m64 = om.from_weights(w, mode="f64")
    assert m32.ew_dtype == np.float32
    k = rng.standard_normal((9, 2, 8))
    v = rng.standard_normal((9, 2, 8))
    qq = rng.standard_normal((9, 4, 8))
    a32 = om.attention(m32, qq, k, v, np.arange(9), np.arange(9))
    a64 = om.attention(m64, qq, k, v, np.arange(9), np.arange(9))
    assert np.max(np.abs(a32 - a64)) < 1e-5 and np.max(np.abs(a32 - a64)) > 0
