"""FP64 chunked (WY / UT) evaluation of the KDA recurrence -- TEST INFRASTRUCTURE ONLY.

This is the second, independent FP64 evaluation used to pin the token oracle.
It follows the seven per-chunk steps listed in "FlashInfer PR #4262: CAKE KDA
Prefill Highlights", section 2 ("Fully fused M128 recurrent pipeline"), and
the fixed exponent anchor of section 1 ("Chunk 32 with a fixed exponent
anchor"), written in plain NumPy with no blocking beyond the chunk itself.

Derivation (so a reader can check it against the recurrence).  Inside one
chunk of L tokens starting from state S0, write Gamma_r = sum_{s<=r} g_s
(inclusive, per channel).  Unrolling
    S_r = Diag(e^{g_r}) S_{r-1} + k_r u_r^T,  u_r = b_r (v_r - S_{r-1}^T Diag(e^{g_r}) k_r)
gives
    S_r = Diag(e^{Gamma_r}) S0 + sum_{s<=r} Diag(e^{Gamma_r - Gamma_s}) k_s u_s^T.
Substituting into u_r:
    u_r + b_r sum_{s<r} (sum_c k_rc k_sc e^{Gamma_rc - Gamma_sc}) u_s
        = b_r (v_r - (k_r * e^{Gamma_r})^T S0)
i.e. (I + A) U = Diag(b) (V - Kg S0) with A strictly lower triangular, so
    U   = T Diag(b) (V - Kg S0),           T = (I + A)^{-1}      (steps 2, 3, 5)
    O   = scale (Qg S0 + M U),              M_rs = sum_c q_rc k_sc e^{Gamma_rc-Gamma_sc}, s<=r
    S_L = Diag(e^{Gamma_L}) S0 + K_r^T U,   K_r[s] = k_s * e^{Gamma_L - Gamma_s}   (steps 4, 6)
where Kg[r] = k_r * e^{Gamma_r} and Qg[r] = q_r * e^{Gamma_r}.  The last two
lines are the note's concatenated update [S_new | O] = [S_d | O_0] + U [K_r | M^T]
written with the state as dk x dv.

Pairwise factors e^{Gamma_r - Gamma_s} can be formed three ways (``mode``):
  "plain"    -- directly, e^{Gamma_r - Gamma_s}.
  "anchored" -- as 2^{G_r - C} * 2^{C - G_s} with G = log2(e) Gamma and the fixed
                anchor C = 16 * lower_bound * log2(e) (section 1); the anchor
                cancels exactly.
  "split16"  -- per 16-token half: diagonal 16x16 blocks anchored at the prefix
                before the half plus 8b, off-diagonal blocks factored through
                the prefix at the split point.  Used when 16|b| exceeds the
                bf16 exponent range (the "ordinary SafeGate" 16-token blocks of
                section 1).
``audit`` (a dict, optional) receives the largest and smallest log2 exponent
of every operand factor formed, so the range claims of section 1 can be
tested.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.4426950408889634

__all__ = ["chunked_prefill", "anchor_constant", "LOG2E"]


def anchor_constant(lower_bound: float) -> float:
    """C = 16 * lower_bound * log2(e) (section 1 of the CAKE prefill note)."""
    return 16.0 * lower_bound * LOG2E


def _note(audit, key, exps):
    if audit is None or exps.size == 0:
        return
    lo, hi = float(np.min(exps)), float(np.max(exps))
    old = audit.get(key)
    audit[key] = (min(lo, old[0]), max(hi, old[1])) if old else (lo, hi)


def _pairwise(left, right, G, mode, lower_bound, audit):
    """sum_c left[r,c] right[s,c] 2^{G[r,c]-G[s,c]} for all r, s (no masking).

    ``left``/``right`` are [L, d]; G is the log2-domain inclusive prefix [L, d].
    """
    L = G.shape[0]
    if mode == "plain":
        E = np.exp2(G[:, None, :] - G[None, :, :])          # [r, s, c]
        return np.einsum("rc,sc,rsc->rs", left, right, E)
    if mode == "anchored":
        C = anchor_constant(lower_bound)
        _note(audit, "anchored", np.concatenate([(G - C).ravel(), (C - G).ravel()]))
        a = left * np.exp2(G - C)
        b = right * np.exp2(C - G)
        return a @ b.T
    if mode == "split16":
        b8 = 8.0 * lower_bound * LOG2E
        out = np.zeros((L, L))
        for r0 in range(0, L, 16):
            r1 = min(r0 + 16, L)
            base = G[r0 - 1] if r0 > 0 else np.zeros(G.shape[1])
            Ch = base + b8
            _note(audit, "split16_diag",
                  np.concatenate([(G[r0:r1] - Ch).ravel(), (Ch - G[r0:r1]).ravel()]))
            out[r0:r1, r0:r1] = (left[r0:r1] * np.exp2(G[r0:r1] - Ch)) @ (
                right[r0:r1] * np.exp2(Ch - G[r0:r1])).T
            for s0 in range(0, r0, 16):
                split = G[r0 - 1]
                ea = G[r0:r1] - split
                eb = split - G[s0:s0 + 16]
                _note(audit, "split16_off", np.concatenate([ea.ravel(), eb.ravel()]))
                out[r0:r1, s0:s0 + 16] = (left[r0:r1] * np.exp2(ea)) @ (
                    right[s0:s0 + 16] * np.exp2(eb)).T
        return out
    raise ValueError(f"unknown mode {mode!r}")


def _unit_lower_inverse(A):
    """(I + A)^{-1} for strictly lower-triangular A, by forward substitution."""
    L = A.shape[0]
    T = np.zeros((L, L))
    for r in range(L):
        T[r, r] = 1.0
        for s in range(r):
            # row r of (I + A) T = e_r  =>  T[r, s] = -sum_{m<r} A[r, m] T[m, s]
            T[r, s] = -np.dot(A[r, s:r], T[s:r, s])
    return T


def chunk_step(S0, q, k, v, g, beta, scale, mode="plain", lower_bound=None, audit=None):
    """One chunk of L tokens: returns (O [L, dv], S_L [dk, dv])."""
    L = q.shape[0]
    Gamma = np.cumsum(g, axis=0)                       # inclusive prefix (natural log)
    G = Gamma * LOG2E                                  # log2 domain
    lower = np.tril(np.ones((L, L), dtype=bool))
    strict = np.tril(np.ones((L, L), dtype=bool), -1)
    M = np.where(lower, _pairwise(q, k, G, mode, lower_bound, audit), 0.0)
    A = np.where(strict, _pairwise(k, k, G, mode, lower_bound, audit), 0.0) * beta[:, None]
    T = _unit_lower_inverse(A)
    decay = np.exp(Gamma)                              # e^{Gamma_r}
    Kg = k * decay
    Qg = q * decay
    U = T @ (beta[:, None] * (v - Kg @ S0))
    O = scale * (Qg @ S0 + M @ U)
    Kr = k * np.exp(Gamma[-1][None, :] - Gamma)
    S1 = np.exp(Gamma[-1])[:, None] * S0 + Kr.T @ U
    return O, S1


def chunked_prefill(q, k, v, g, beta, cu_seqlens, scale, initial_state=None, chunk=32,
                    mode="plain", lower_bound=None, audit=None):
    """Chunked FP64 prefill over packed sequences; same layouts as ``oracle.prefill``.

    The last chunk of a sequence may be shorter than ``chunk``.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    if mode != "plain" and (lower_bound is None or not math.isfinite(lower_bound)):
        raise ValueError("anchored modes need a finite lower_bound")
    out = np.zeros((T, H, dv))
    final = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = (np.zeros((dk, dv)) if initial_state is None
                 else np.array(initial_state[n, h], dtype=np.float64))
            for t0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                t1 = min(t0 + chunk, int(cu[n + 1]))
                O, S = chunk_step(S, q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], g[t0:t1, h],
                                  beta[t0:t1, h], scale, mode, lower_bound, audit)
                out[t0:t1, h] = O
            final[n, h] = S
    return out, final
