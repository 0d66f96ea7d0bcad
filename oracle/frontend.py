"""FP64 input front-end of the KDA step -- TEST INFRASTRUCTURE ONLY (part of the oracle).

The kernels' callers may hand over raw model quantities instead of the gated,
normalised ones the recurrence consumes.  "flashinfer PR #5551: Kimi K3 TP12
H=8 fused KDA decode" lists the decode scalars as H, rows, use_lower_bound,
lower_bound_log2 and norm_eps, and tests "softplus and lower-bound gates";
the PR #5565 / #5573 benchmark notes take beta through a sigmoid of logits and
call the unbounded gate "softplus".  Readings taken here (the pages print no
formulas for them):

* lower-bound gate: g = lower_bound * sigmoid(a) (natural-log decay in
  (lower_bound, 0); lower_bound < 0 given in natural-log units),
* softplus gate:    g = -softplus(a) = -log(1 + exp(a)) (unbounded below),
* beta from logits: beta = sigmoid(b),
* q, k L2 norm:     x / sqrt(sum_c x_c^2 + norm_eps) over the 128 channels of
  one (token, head); a zero vector with norm_eps = 0 stays zero.

Each function is the plain definition in double precision, written in a form
that neither overflows nor cancels (so that tests can use extreme inputs).
Pinned in ``tests/test_oracle_pins.py`` by closed forms and identities.
"""
from __future__ import annotations

import numpy as np

GATE_LOG, GATE_LOWER_BOUND, GATE_SOFTPLUS = 0, 1, 2


def sigmoid(x) -> np.ndarray:
    """1 / (1 + e^-x), evaluated through e^-|x| (no overflow for any x)."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x) -> np.ndarray:
    """log(1 + e^x) = max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gate(a, mode: int, lower_bound: float = 0.0) -> np.ndarray:
    """Natural-log decay g from the caller's gate input for `mode`."""
    a = np.asarray(a, dtype=np.float64)
    if mode == GATE_LOG:
        return a.copy()
    if mode == GATE_LOWER_BOUND:
        return float(lower_bound) * sigmoid(a)
    if mode == GATE_SOFTPLUS:
        return -softplus(a)
    raise ValueError(f"unknown gate mode {mode}")


def l2_normalize(x, eps: float) -> np.ndarray:
    """x / sqrt(sum x^2 + eps) along the last axis (the 128 channels); a zero
    vector with eps = 0 stays zero (reading: no 0/0)."""
    x = np.asarray(x, dtype=np.float64)
    d = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))
    return np.divide(x, d, out=np.zeros_like(x), where=d > 0)


def apply(q, k, g_in, beta_in, *, gate_mode=GATE_LOG, lower_bound=0.0, beta_logits=False,
          normalize_qk=False, norm_eps=0.0):
    """(q, k, g, beta) as the recurrence consumes them, in float64.

    q, k, g_in: [..., 128]; beta_in: [...] (the same leading shape)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if normalize_qk:
        q, k = l2_normalize(q, norm_eps), l2_normalize(k, norm_eps)
    g = gate(g_in, gate_mode, lower_bound)
    beta = sigmoid(beta_in) if beta_logits else np.asarray(beta_in, dtype=np.float64).copy()
    return q, k, g, beta
