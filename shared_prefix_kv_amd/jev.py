"""Thin Python binding of libjev.so (include/jev.h).

Argument marshalling only: every step of scoring runs in the HIP kernels behind
the C ABI.  PyTorch is used for device memory (weights, KV pool, workspace,
outputs) and for the current HIP stream.  If the library has not been built,
importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# JEV_LIB selects another build of the same library (the sanitizer build for
# the CPU tests); the default is the in-tree libjev.so
LIB_PATH = os.environ.get("JEV_LIB") or os.path.join(_HERE, "lib", "libjev.so")

JEV_OK, JEV_EINVAL, JEV_ENOMEM, JEV_EHANDLE, JEV_EHIP, JEV_ESTATE, JEV_EPENDING = range(7)
JEV_DTYPE_F32, JEV_DTYPE_BF16 = 0, 1
JEV_TAP_ATTN, JEV_TAP_RESID = 0, 1
JEV_ANSWER_NOUL, JEV_ANSWER_CHOICE, JEV_ANSWER_SCORE = 0, 1, 2
JEV_PLAN_DEPTH, JEV_PLAN_CANDIDATE_FIRST = 0, 1
JEV_CACHE_RELEASE, JEV_CACHE_LRU = 0, 1
JEV_SCHED_QUEUED, JEV_SCHED_ACTIVE, JEV_SCHED_FINISHED = 0, 1, 2
JEV_DEBUG_POISON_FREED_PAGES, JEV_DEBUG_TIME_CALLS, JEV_DEBUG_FULL_LAST_LAYER = 1, 2, 4
JEV_CALL_NONE, JEV_CALL_PREFILL, JEV_CALL_BRANCHES, JEV_CALL_CANDIDATES, JEV_CALL_SCHED_STEP = 0, 1, 2, 3, 4
_NAMES = {0: "JEV_OK", 1: "JEV_EINVAL", 2: "JEV_ENOMEM", 3: "JEV_EHANDLE", 4: "JEV_EHIP", 5: "JEV_ESTATE",
          6: "JEV_EPENDING"}

EXPORTED = ["jev_workspace_bytes", "jev_kv_pool_bytes", "jev_create", "jev_destroy", "jev_prefill_prefix",
            "jev_score_branches", "jev_score_branches_noalloc", "jev_score_candidates", "jev_free_pages", "jev_plan", "jev_page_table",
            "jev_match", "jev_stats", "jev_debug_tap", "jev_profile", "jev_profile_rows", "jev_profile_read", "jev_answers",
            "jev_set_plan_mode", "jev_set_cache_policy", "jev_sched_create", "jev_sched_destroy",
            "jev_sched_submit", "jev_sched_step", "jev_sched_status", "jev_sched_result", "jev_last_error",
            "jev_set_debug", "jev_limits", "jev_set_gemm_variant", "jev_set_round_invariant"]
KERNELS = ["embed", "rmsnorm", "qkv", "attn", "merge", "oproj", "readout"]


class JevError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("max_positions", ctypes.c_int32), ("max_round_tokens", ctypes.c_int32)]


class WeightsC(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("unembed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", ctypes.POINTER(ctypes.c_void_p)), ("wq", ctypes.POINTER(ctypes.c_void_p)),
                ("wk", ctypes.POINTER(ctypes.c_void_p)), ("wv", ctypes.POINTER(ctypes.c_void_p)),
                ("wo", ctypes.POINTER(ctypes.c_void_p))]


class LaunchRecord(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double), ("ms", ctypes.c_float)]


class Stats(ctypes.Structure):
    _fields_ = [("logical_tokens", ctypes.c_int64), ("computed_tokens", ctypes.c_int64),
                ("cached_tokens", ctypes.c_int64), ("rounds", ctypes.c_int32), ("pages_in_use", ctypes.c_int32),
                ("pages_total", ctypes.c_int32), ("resident_prefixes", ctypes.c_int32), ("calls", ctypes.c_int64),
                ("cached_prefixes", ctypes.c_int32), ("cached_pages", ctypes.c_int32), ("evictions", ctypes.c_int64),
                ("last_call_kind", ctypes.c_int32), ("debug_flags", ctypes.c_uint32),
                ("last_prepare_ns", ctypes.c_int64), ("last_enqueue_ns", ctypes.c_int64),
                ("last_prefill_ms", ctypes.c_double), ("last_branch_ms", ctypes.c_double)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class Limits(ctypes.Structure):
    _fields_ = [("page_tokens", ctypes.c_int32), ("min_labels", ctypes.c_int32), ("max_labels", ctypes.c_int32),
                ("max_positions", ctypes.c_int32), ("max_round_tokens", ctypes.c_int32), ("n_pages", ctypes.c_int32),
                ("split_k_rows", ctypes.c_int32), ("max_tile_pages", ctypes.c_int32),
                ("noalloc_scratch_bytes", ctypes.c_int64), ("noalloc_partial_rows", ctypes.c_int64),
                ("workspace_partial_rows", ctypes.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m shared_prefix_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.jev_workspace_bytes.argtypes = [P(ModelDesc)]
        L.jev_workspace_bytes.restype = ctypes.c_size_t
        L.jev_kv_pool_bytes.argtypes = [P(ModelDesc), i32]
        L.jev_kv_pool_bytes.restype = ctypes.c_size_t
        L.jev_create.argtypes = [P(ModelDesc), P(WeightsC), vp, i32, vp, ctypes.c_size_t, P(vp)]
        L.jev_destroy.argtypes = [vp]
        L.jev_prefill_prefix.argtypes = [vp, i32, P(i64), P(i32), P(i64), P(i64), vp]
        L.jev_score_branches.argtypes = [vp, i32, P(i64), P(i32), P(i64), P(i32), P(i64), vp, vp]
        L.jev_score_branches_noalloc.argtypes = [vp, i32, P(i64), P(i32), P(i64), P(i32), P(i64), vp, vp]
        L.jev_score_candidates.argtypes = [vp, i32, P(i32), P(i64), P(i32), P(i64), vp, vp]
        L.jev_free_pages.argtypes = [vp, i32, P(i64)]
        L.jev_plan.argtypes = [vp, i32, P(i32), P(i64), P(i32), i64, P(i64)]
        L.jev_page_table.argtypes = [vp, i64, P(i32), P(i32), i32, P(i32)]
        L.jev_match.argtypes = [vp, P(i32), i64, P(i64), P(i64)]
        L.jev_stats.argtypes = [vp, P(Stats)]
        L.jev_debug_tap.argtypes = [vp, i32, i32, vp, i64]
        L.jev_profile.argtypes = [vp, ctypes.c_uint32]
        L.jev_profile_rows.argtypes = [vp, ctypes.c_uint32, i64]
        L.jev_profile_read.argtypes = [vp, P(LaunchRecord), i64, P(i64)]
        L.jev_set_plan_mode.argtypes = [vp, i32]
        L.jev_set_cache_policy.argtypes = [vp, i32]
        L.jev_answers.argtypes = [i32, P(ctypes.c_float), P(i64), P(i32), P(ctypes.c_double), P(i32),
                                  P(ctypes.c_double)]
        L.jev_sched_create.argtypes = [vp, P(vp)]
        L.jev_sched_destroy.argtypes = [vp]
        L.jev_sched_submit.argtypes = [vp, i32, P(i32), P(i64), P(i32), P(i64), P(i64)]
        L.jev_sched_step.argtypes = [vp, vp, P(i32), i64, P(i64)]
        L.jev_sched_status.argtypes = [vp, i64, P(i32)]
        L.jev_sched_result.argtypes = [vp, i64, P(ctypes.c_float), i64]
        L.jev_last_error.restype = ctypes.c_char_p
        L.jev_set_debug.argtypes = [vp, ctypes.c_uint32]
        L.jev_limits.argtypes = [vp, P(Limits)]
        L.jev_set_gemm_variant.argtypes = [i32, i32, i32]
        L.jev_set_round_invariant.argtypes = [vp, i32]
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != JEV_OK:
        raise JevError(rc, lib().jev_last_error().decode())


def set_gemm_variant(large: int = 0, splits: int = 0, bn: int = 0) -> None:
    """Projection kernel variant for measurement (process-wide; see jev.h)."""
    _check(lib().jev_set_gemm_variant(int(large), int(splits), int(bn)))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _segments(segs: Sequence[Sequence[int]]) -> Tuple[np.ndarray, np.ndarray]:
    lens = [len(s) for s in segs]
    off = np.zeros(len(segs) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    flat = _i32(np.concatenate([np.asarray(s, dtype=np.int32) for s in segs]) if segs else [])
    return flat, off


def make_desc(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, vocab, dtype, rope_theta, rms_eps,
              max_positions, max_round_tokens) -> ModelDesc:
    return ModelDesc(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, vocab,
                     JEV_DTYPE_BF16 if dtype == "bf16" else JEV_DTYPE_F32, rope_theta, rms_eps,
                     max_positions, max_round_tokens)


def upload_weights(w, device="cuda:0") -> dict:
    """Host weights (uint16 bf16 patterns or float32 numpy arrays, [out, in]
    layout) -> device tensors of the storage dtype."""
    import torch

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return {"embed": dev(w.embed), "unembed": dev(w.unembed), "final_norm": dev(w.final_norm),
            "attn_norm": [dev(a) for a in w.attn_norm], "wq": [dev(a) for a in w.wq],
            "wk": [dev(a) for a in w.wk], "wv": [dev(a) for a in w.wv], "wo": [dev(a) for a in w.wo]}


def answers(probs, label_offsets, kinds):
    """jev_answers: per branch (value, choice, confidence) from host label
    distributions.  probs: float32 values (numpy, list or a torch tensor, which
    is copied to the host); label_offsets: n+1 int64; kinds: n JEV_ANSWER_*.
    Returns three numpy arrays: value (float64), choice (int32), confidence
    (float64)."""
    if hasattr(probs, "detach"):
        probs = probs.detach().cpu().numpy()
    p = np.ascontiguousarray(np.asarray(probs, dtype=np.float32))
    off = _i64(label_offsets)
    k = _i32(kinds)
    n = len(k)
    if len(off) != n + 1:
        raise ValueError("label_offsets needs n + 1 entries")
    value = np.zeros(n, dtype=np.float64)
    choice = np.zeros(n, dtype=np.int32)
    conf = np.zeros(n, dtype=np.float64)
    if n:
        _check(lib().jev_answers(n, _ptr(p, ctypes.c_float), _ptr(off, ctypes.c_int64), _ptr(k, ctypes.c_int32),
                                 _ptr(value, ctypes.c_double), _ptr(choice, ctypes.c_int32),
                                 _ptr(conf, ctypes.c_double)))
    return value, choice, conf


def _current_stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Context:
    """A jev context.  ``weights=None`` creates a planning-only context."""

    def __init__(self, desc: ModelDesc, n_pages: int, weights: Optional[dict] = None, device="cuda:0"):
        L = lib()
        self.desc = desc
        self.n_pages = n_pages
        self._keep = []
        ctx = ctypes.c_void_p()
        if weights is None:
            _check(L.jev_create(ctypes.byref(desc), None, None, n_pages, None, 0, ctypes.byref(ctx)))
        else:
            import torch
            pool_bytes = L.jev_kv_pool_bytes(ctypes.byref(desc), n_pages)
            ws_bytes = L.jev_workspace_bytes(ctypes.byref(desc))
            if pool_bytes == 0 or ws_bytes == 0:
                raise JevError(JEV_EINVAL, "unsupported model description")
            self.pool = torch.empty(pool_bytes, dtype=torch.uint8, device=device)
            self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
            n = desc.n_layers
            arr = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])
            per_layer = [arr(weights[k]) for k in ("attn_norm", "wq", "wk", "wv", "wo")]
            self._keep += per_layer
            wc = WeightsC(weights["embed"].data_ptr(), weights["unembed"].data_ptr(),
                          weights["final_norm"].data_ptr(),
                          *[ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)) for a in per_layer])
            self.weights = weights
            _check(L.jev_create(ctypes.byref(desc), ctypes.byref(wc), self.pool.data_ptr(), n_pages,
                                self.workspace.data_ptr(), ws_bytes, ctypes.byref(ctx)))
        self.ctx = ctx

    def close(self) -> None:
        if self.ctx:
            # schedulers belong to the context: destroy them first
            for ref in getattr(self, "_scheds", []):
                sch = ref()
                if sch is not None:
                    sch.close()
            _check(lib().jev_destroy(self.ctx))
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ calls
    def prefill_prefix(self, parents: Sequence[int], segments: Sequence[Sequence[int]], stream=None) -> List[int]:
        par = _i64(parents)
        flat, off = _segments(segments)
        out = np.zeros(len(segments), dtype=np.int64)
        _check(lib().jev_prefill_prefix(self.ctx, len(segments), _ptr(par, ctypes.c_int64),
                                        _ptr(flat, ctypes.c_int32), _ptr(off, ctypes.c_int64),
                                        _ptr(out, ctypes.c_int64), stream or self._stream()))
        return [int(h) for h in out]

    def score_branches(self, parents, suffixes, labels, probs=None, stream=None, noalloc=False):
        """Returns (probs device tensor [sum K] float32, label offsets).
        noalloc: call jev_score_branches_noalloc (the caller passes probs)."""
        par = _i64(parents)
        flat, off = _segments(suffixes)
        lflat, loff = _segments(labels)
        probs = self._probs(probs, int(loff[-1]))
        fn = lib().jev_score_branches_noalloc if noalloc else lib().jev_score_branches
        _check(fn(self.ctx, len(suffixes), _ptr(par, ctypes.c_int64), _ptr(flat, ctypes.c_int32),
                  _ptr(off, ctypes.c_int64), _ptr(lflat, ctypes.c_int32), _ptr(loff, ctypes.c_int64),
                  ctypes.c_void_p(probs.data_ptr()), stream or self._stream()))
        return probs, loff

    def score_candidates(self, seqs, labels, probs=None, stream=None):
        flat, off = _segments(seqs)
        lflat, loff = _segments(labels)
        probs = self._probs(probs, int(loff[-1]))
        _check(lib().jev_score_candidates(self.ctx, len(seqs), _ptr(flat, ctypes.c_int32),
                                          _ptr(off, ctypes.c_int64), _ptr(lflat, ctypes.c_int32),
                                          _ptr(loff, ctypes.c_int64), ctypes.c_void_p(probs.data_ptr()),
                                          stream or self._stream()))
        return probs, loff

    def free_pages(self, handles: Sequence[int]) -> None:
        h = _i64(handles)
        _check(lib().jev_free_pages(self.ctx, len(h), _ptr(h, ctypes.c_int64)))

    def set_plan_mode(self, mode: int) -> None:
        """JEV_PLAN_DEPTH or JEV_PLAN_CANDIDATE_FIRST (jev_set_plan_mode)."""
        _check(lib().jev_set_plan_mode(self.ctx, mode))

    def set_cache_policy(self, policy: int) -> None:
        """JEV_CACHE_RELEASE or JEV_CACHE_LRU (jev_set_cache_policy)."""
        _check(lib().jev_set_cache_policy(self.ctx, policy))

    def set_round_invariant(self, on: bool) -> None:
        """Round-invariant numerics (jev_set_round_invariant)."""
        _check(lib().jev_set_round_invariant(self.ctx, int(bool(on))))

    def set_debug(self, flags: int) -> None:
        """JEV_DEBUG_* bit flags (jev_set_debug); 0 turns them off."""
        _check(lib().jev_set_debug(self.ctx, flags))

    def limits(self) -> dict:
        out = Limits()
        _check(lib().jev_limits(self.ctx, ctypes.byref(out)))
        return out.as_dict()

    def plan(self, seqs) -> List[int]:
        flat, off = _segments(seqs)
        n = ctypes.c_int64()
        _check(lib().jev_plan(self.ctx, len(seqs), _ptr(flat, ctypes.c_int32), _ptr(off, ctypes.c_int64), None,
                              0, ctypes.byref(n)))
        out = np.zeros(n.value, dtype=np.int32)
        _check(lib().jev_plan(self.ctx, len(seqs), _ptr(flat, ctypes.c_int32), _ptr(off, ctypes.c_int64),
                              _ptr(out, ctypes.c_int32), n.value, ctypes.byref(n)))
        return [int(v) for v in out]

    def page_table(self, handle: int) -> Tuple[List[int], List[int]]:
        n = ctypes.c_int32()
        rc = lib().jev_page_table(self.ctx, handle, None, None, 0, ctypes.byref(n))
        if rc not in (JEV_OK, JEV_EINVAL) or (rc == JEV_EINVAL and n.value == 0):
            _check(rc)
        pages = np.zeros(n.value, dtype=np.int32)
        valid = np.zeros(n.value, dtype=np.int32)
        _check(lib().jev_page_table(self.ctx, handle, _ptr(pages, ctypes.c_int32), _ptr(valid, ctypes.c_int32),
                                    n.value, ctypes.byref(n)))
        return [int(p) for p in pages], [int(v) for v in valid]

    def match(self, tokens) -> Tuple[int, int]:
        t = _i32(tokens)
        h, m = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().jev_match(self.ctx, _ptr(t, ctypes.c_int32), len(t), ctypes.byref(h), ctypes.byref(m)))
        return h.value, m.value

    def stats(self) -> dict:
        s = Stats()
        _check(lib().jev_stats(self.ctx, ctypes.byref(s)))
        return s.as_dict()

    def debug_tap(self, what: int = 0, layer: int = 0, dst=None) -> None:
        """what: JEV_TAP_ATTN or JEV_TAP_RESID; dst=None removes every tap."""
        if dst is None:
            _check(lib().jev_debug_tap(self.ctx, 0, 0, None, 0))
        else:
            _check(lib().jev_debug_tap(self.ctx, what, layer, ctypes.c_void_p(dst.data_ptr()), dst.shape[0]))

    def profile(self, kinds: Sequence[str] = (), rows: int = 0) -> None:
        """Enables event timing of the named kernels (with rows > 0: of their
        launches of exactly that many rows); () disables and clears."""
        mask = 0
        for k in kinds:
            mask |= 1 << KERNELS.index(k)
        _check(lib().jev_profile_rows(self.ctx, mask, rows))

    def profile_read(self) -> List[dict]:
        n = ctypes.c_int64()
        _check(lib().jev_profile_read(self.ctx, None, 0, ctypes.byref(n)))
        recs = (LaunchRecord * max(1, n.value))()
        _check(lib().jev_profile_read(self.ctx, recs, n.value, ctypes.byref(n)))
        return [{"kernel": KERNELS[r.kind], "layer": r.layer, "rows": r.rows, "flops": r.flops,
                 "bytes": r.bytes, "ms": r.ms} for r in recs[:n.value]]

    # ------------------------------------------------------------------ helpers
    def _stream(self):
        return _current_stream() if hasattr(self, "pool") else None

    def _probs(self, probs, n):
        import torch
        if probs is None:
            if not hasattr(self, "pool"):
                return _NullTensor()
            probs = torch.empty(n, dtype=torch.float32, device=self.pool.device)
        return probs


class Scheduler:
    """Round-level continuous batching on a context (jev_sched_*): submit() from
    any thread, step() from one driver thread, result() once finished."""

    def __init__(self, ctx: Context):
        import weakref
        self.owner = ctx
        s = ctypes.c_void_p()
        _check(lib().jev_sched_create(ctx.ctx, ctypes.byref(s)))
        self.s = s
        self._loff: Dict[int, np.ndarray] = {}
        if not hasattr(ctx, "_scheds"):
            ctx._scheds = []
        ctx._scheds.append(weakref.ref(self))

    def close(self) -> None:
        if self.s:
            _check(lib().jev_sched_destroy(self.s))
            self.s = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, seqs, labels) -> int:
        flat, off = _segments(seqs)
        lflat, loff = _segments(labels)
        t = ctypes.c_int64()
        _check(lib().jev_sched_submit(self.s, len(seqs), _ptr(flat, ctypes.c_int32), _ptr(off, ctypes.c_int64),
                                      _ptr(lflat, ctypes.c_int32), _ptr(loff, ctypes.c_int64), ctypes.byref(t)))
        self._loff[t.value] = loff
        return t.value

    def step(self, stream=None, want_plan: bool = False) -> Optional[List[int]]:
        """One round; with want_plan, the plan it was taken from (jev_plan format)."""
        n = ctypes.c_int64()
        st = stream or self.owner._stream()
        if not want_plan:
            _check(lib().jev_sched_step(self.s, st, None, 0, ctypes.byref(n)))
            return None
        cap = 1 << 20
        buf = np.zeros(cap, dtype=np.int32)
        _check(lib().jev_sched_step(self.s, st, _ptr(buf, ctypes.c_int32), cap, ctypes.byref(n)))
        return [int(v) for v in buf[:n.value]]

    def status(self, ticket: int) -> int:
        st = ctypes.c_int32()
        _check(lib().jev_sched_status(self.s, ticket, ctypes.byref(st)))
        return st.value

    def result(self, ticket: int) -> List[np.ndarray]:
        """Per candidate, its label probabilities (host float32)."""
        loff = self._loff[ticket]
        out = np.zeros(int(loff[-1]), dtype=np.float32)
        _check(lib().jev_sched_result(self.s, ticket, _ptr(out, ctypes.c_float), len(out)))
        del self._loff[ticket]
        return [out[loff[i]:loff[i + 1]] for i in range(len(loff) - 1)]


class _NullTensor:
    """Stands in for an output on a planning-only context (calls fail first)."""

    def data_ptr(self):
        return 0
