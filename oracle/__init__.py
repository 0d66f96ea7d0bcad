"""FP64 CPU oracle for the KDA gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU product path
(``kimi_delta_attention_prefill_amd``) never imports it, and the two share no
code: the only module both sides use is the seeded input generator, which
holds none of the method's arithmetic.

Contents
--------
``prefill`` / ``decode``
    ctypes front-ends to ``kda_oracle.c``: the plain token-by-token
    recurrence S_t = (I - b_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + b_t k_t v_t^T,
    o_t = scale S_t^T q_t, evaluated in double (the recurrence whose chunked
    form "FlashInfer PR #4262: CAKE KDA Prefill Highlights", section 2,
    computes).  Inputs are read as exact doubles from their bf16/fp32 values.
``chunked``
    An independent FP64 evaluation of the same map in the chunked (WY / UT)
    form of section 2 of that note, with the fixed exponent anchor of
    section 1.  It exists to pin the token oracle (it is a different
    algorithm), not to stand in for it.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, exact special cases, a hand-derived worked example and the
chunked-form cross-check).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build, library_path

__all__ = ["prefill", "decode", "build", "library_path", "default_threads"]

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(
        os.path.join(os.path.dirname(__file__), "kda_oracle.c")
    ):
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.kda_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, ip, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp, dp,
                                       ctypes.c_int]
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_prefill_snapshots.argtypes = [dp, dp, dp, dp, dp, ip, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_double, dp,
                                                 dp, dp, ctypes.c_int64, dp, ctypes.c_int]
    lib.kda_oracle_prefill_snapshots.restype = ctypes.c_int
    lib.kda_oracle_decode.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_int64, ip, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, dp,
                                      ctypes.c_int]
    lib.kda_oracle_decode.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses by default: the host's usable cores, capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16/fp32 -> fp64 widening is exact
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prefill(q, k, v, g, beta, cu_seqlens, scale, initial_state=None, want_final=True,
            threads=None, snapshot_every=None):
    """Token-serial FP64 prefill over packed sequences.

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; cu_seqlens: [N+1];
    initial_state: [N, H, dk, dv] or None (zeros).
    Returns (out [T, H, dv] float64, final_state [N, H, dk, dv] float64 or None),
    and with ``snapshot_every = I`` also a list over sequences of the states
    after I, 2I, ... tokens ([floor(len_n / I), H, dk, dv] float64 each).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    cu = np.ascontiguousarray(np.asarray(
        cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk) and v.shape == (T, H, dv)
    assert beta.shape == (T, H) and int(cu[-1]) == T
    s0 = _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    out = np.zeros((T, H, dv), dtype=np.float64)
    s1 = np.zeros((N, H, dk, dv), dtype=np.float64) if want_final else None
    every = int(snapshot_every or 0)
    counts = [int(cu[n + 1] - cu[n]) // every for n in range(N)] if every else []
    snaps = np.zeros((max(1, sum(counts)), H, dk, dv), dtype=np.float64) if every else None
    rc = _load().kda_oracle_prefill_snapshots(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, H, dk, dv, float(scale),
        _ptr(s0), _ptr(s1), _ptr(out), every, _ptr(snaps), int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"kda_oracle_prefill failed with code {rc}")
    if not every:
        return out, s1
    per_seq, at = [], 0
    for cnt in counts:
        per_seq.append(snaps[at:at + cnt])
        at += cnt
    return out, s1, per_seq


def decode(q, k, v, g, beta, pool, slot_indices, scale, threads=None):
    """One T=1 step per row over a slot-indexed pool (updated copy returned).

    q, k, g: [rows, H, dk]; v: [rows, H, dv]; beta: [rows, H];
    pool: [num_slots, H, dk, dv]; slot_indices: [rows] (negative = skip row).
    Returns (out [rows, H, dv] float64, new_pool float64).  The input pool is
    not modified.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    pool = np.array(_f64(pool), dtype=np.float64, copy=True)
    slots = np.ascontiguousarray(np.asarray(
        slot_indices.cpu().numpy() if hasattr(slot_indices, "cpu") else slot_indices,
        dtype=np.int64))
    rows, H, dk = q.shape
    dv = v.shape[2]
    out = np.zeros((rows, H, dv), dtype=np.float64)
    rc = _load().kda_oracle_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(pool), pool.shape[0],
        slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows, H, dk, dv, float(scale),
        _ptr(out), int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"kda_oracle_decode failed with code {rc}")
    return out, pool
