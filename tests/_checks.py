"""Tolerance checks shared by the GPU parity tests.

Bounds (the floating-point tolerance of the KDA path, written out):

* prefill / FP32-state decode output o (bf16):
      |o_gpu - o_ref| <= 2e-2 * RMS(o_ref) + halfulp_bf16(max(|o_gpu|, |o_ref|))
  elementwise.  RMS is over all compared entries.  The half-ulp term is the
  rounding every bf16 output carries even when computed exactly: the outputs
  are heavy-tailed (max/RMS ~ 15 on the T=8192 workload), so bf16 rounding
  of the exact result alone reaches ~0.04 RMS at the largest entries and a
  bare 2e-2 RMS bound could not be met by any bf16-output implementation.
* final state (fp32):  max |S_gpu - S_ref| <= 1e-2 * RMS(S_ref).
* BF16-state decode, pool after the step (stored in bf16):
      |S_gpu - S_ref| <= halfulp_bf16(max(|S_gpu|, |S_ref|)) + 1e-3 * RMS(S_ref)
  i.e. one bf16 rounding of the exact update plus a small computational
  term; the reference starts from the bf16-stored state read as exact.
"""
from __future__ import annotations

import numpy as np
import torch

OUT_TOL = 2e-2
STATE_TOL = 1e-2
BF16_STATE_TOL = 1e-3


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def halfulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half of a bf16 ulp at |x| (exact: 2^(floor(log2|x|) - 8)); 0 at 0."""
    m, e = np.frexp(np.abs(x))           # |x| = m 2^e, m in [0.5, 1)
    h = np.ldexp(np.ones_like(m), e - 9)
    return np.where(x == 0, 0.0, h)


def rms(x) -> float:
    x = _f64(x)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def check_out(gpu, ref, tol=OUT_TOL, what="out"):
    g, r = _f64(gpu), _f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    R = rms(r)
    excess = np.abs(g - r) - halfulp_bf16(np.maximum(np.abs(g), np.abs(r)))
    worst = float(np.max(excess, initial=0.0))
    rel_l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    assert worst <= tol * R + 1e-30, (
        f"{what}: max(|err| - halfulp) = {worst:.3e} > {tol} * RMS = {tol * R:.3e} "
        f"(rel-L2 {rel_l2:.2e})")
    return dict(max_excess_over_rms=worst / R if R else 0.0, rel_l2=rel_l2)


def check_state(gpu, ref, tol=STATE_TOL, what="state"):
    g, r = _f64(gpu), _f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    R = rms(r)
    err = float(np.max(np.abs(g - r), initial=0.0))
    rel_l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    assert err <= tol * R + 1e-30, (
        f"{what}: max|err| = {err:.3e} > {tol} * RMS = {tol * R:.3e} (rel-L2 {rel_l2:.2e})")
    return dict(max_err_over_rms=err / R if R else 0.0, rel_l2=rel_l2)


def check_bf16_state(gpu, ref, tol=BF16_STATE_TOL, what="bf16 state"):
    g, r = _f64(gpu), _f64(ref)
    assert g.shape == r.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    R = rms(r)
    excess = np.abs(g - r) - halfulp_bf16(np.maximum(np.abs(g), np.abs(r)))
    worst = float(np.max(excess, initial=0.0))
    assert worst <= tol * R + 1e-30, (
        f"{what}: max(|err| - halfulp) = {worst:.3e} > {tol} * RMS = {tol * R:.3e}")
    return dict(max_excess_over_rms=worst / R if R else 0.0)
