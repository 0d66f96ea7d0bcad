"""Pins of the FP64 oracle against facts fixed by the mathematics (CPU only).

Each test names the mistake it would catch.  Nothing here calls the GPU path.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.chunked import chunked_prefill, anchor_constant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG_SEED = 1234


def _rand_case(lengths, H, dk=16, dv=12, lb=-5.0, init=True, seed=RNG_SEED, beta=None, g=None):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    gg = lb / (1.0 + np.exp(-rng.standard_normal((T, H, dk)))) if g is None else g
    bb = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H)))) if beta is None else beta
    s0 = 0.3 * rng.standard_normal((len(lengths), H, dk, dv)) if init else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(q=q, k=k, v=v, g=gg, beta=bb, cu=cu, s0=s0)


def _run(c, scale=0.25, threads=4):
    return oracle.prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], scale,
                          c["s0"], threads=threads)


def _close(a, b, rtol=1e-12):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert a.shape == b.shape
    assert np.max(np.abs(a - b), initial=0.0) <= rtol * scale, np.max(np.abs(a - b))


# --------------------------------------------------------------- worked example
def test_hand_derived_two_steps():
    """Exact two-step example derived by hand (decay order, erase, write, scale,
    post-update read, state orientation: any slip changes a printed decimal)."""
    with open(os.path.join(GOLDEN, "hand_two_steps_dk2.json")) as f:
        gold = json.load(f)
    ln2 = math.log(2.0)
    g = np.array([[0.0, -ln2], [-ln2, 0.0]])[:, None, :]
    q = np.array(gold["q"])[:, None, :]
    k = np.array(gold["k"])[:, None, :]
    v = np.array(gold["v"])[:, None, :]
    beta = np.array(gold["beta"])[:, None]
    s0 = np.array(gold["S0"])[None, None]
    out, fin = oracle.prefill(q, k, v, g, beta, [0, 2], gold["scale"], s0)
    np.testing.assert_allclose(out[:, 0], gold["expected_out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], gold["expected_final_state"], rtol=0, atol=1e-14)


def test_hand_derived_decode_matches():
    """The same first step through the slot-indexed decode entry (slot 1 of 3)."""
    with open(os.path.join(GOLDEN, "hand_two_steps_dk2.json")) as f:
        gold = json.load(f)
    pool = np.zeros((3, 1, 2, 2))
    pool[1, 0] = gold["S0"]
    pool[0, 0] = 7.0
    pool[2, 0] = -7.0
    out, newpool = oracle.decode(np.array(gold["q"][:1])[:, None], np.array(gold["k"][:1])[:, None],
                                 np.array(gold["v"][:1])[:, None],
                                 np.array([[[0.0, -math.log(2.0)]]]),
                                 np.array([[gold["beta"][0]]]), pool, [1], gold["scale"])
    np.testing.assert_allclose(out[0, 0], gold["expected_out"][0], atol=1e-14)
    np.testing.assert_allclose(newpool[1, 0], [[0.76, 0.86], [1.18, 0.48]], atol=1e-14)
    assert np.all(newpool[0] == 7.0) and np.all(newpool[2] == -7.0)  # other slots untouched
    assert np.all(pool[1, 0] == gold["S0"])                            # input pool not modified


# ---------------------------------------------------------------- closed forms
def test_beta_zero_is_pure_decay():
    """I1: beta = 0 => S_t = Diag(e^{Gamma_t}) S0 and o_t = scale (Diag(e^{Gamma_t}) S0)^T q_t.
    Catches exp vs exp2, a missing or doubled decay, a wrong prefix, a dropped S0."""
    c = _rand_case([5, 9, 1], H=2, beta=None)
    c["beta"] = np.zeros_like(c["beta"])
    scale = 0.3
    out, fin = _run(c, scale)
    for n in range(3):
        t0, t1 = c["cu"][n], c["cu"][n + 1]
        for h in range(2):
            gam = np.zeros(c["q"].shape[2])
            for t in range(t0, t1):
                gam = gam + c["g"][t, h]
                St = np.exp(gam)[:, None] * c["s0"][n, h]
                _close(out[t, h], scale * St.T @ c["q"][t, h])
            _close(fin[n, h], np.exp(gam)[:, None] * c["s0"][n, h])


def test_orthonormal_overwrite():
    """I2: g = 0, beta = 1, orthonormal keys => S_T = (I - K K^T) S0 + K V^T, and
    reading with q_t = k_t returns scale * v_t.  Catches a wrong erase (sign, missing
    beta, k vs q), a pre-update read and a missing scale."""
    rng = np.random.default_rng(7)
    dk, dv, T = 24, 10, 20
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Q[:, :T].T                                   # T orthonormal keys
    v = rng.standard_normal((T, 1, dv))
    s0 = rng.standard_normal((1, 1, dk, dv))
    q = K[:, None, :].copy()
    scale = 0.7
    out, fin = oracle.prefill(q, K[:, None, :], v, np.zeros((T, 1, dk)), np.ones((T, 1)),
                              [0, T], scale, s0)
    P = np.eye(dk) - K.T @ K
    _close(fin[0, 0], P @ s0[0, 0] + K.T @ v[:, 0])
    _close(out[:, 0], scale * v[:, 0])


def test_basis_keys_set_rows():
    """I2 with standard-basis keys: writing e_c sets row c of S to v exactly."""
    dk, dv = 8, 5
    perm = [3, 0, 6]
    k = np.zeros((3, 1, dk))
    for t, c in enumerate(perm):
        k[t, 0, c] = 1.0
    v = np.arange(15, dtype=float).reshape(3, 1, dv) - 4.0
    s0 = np.full((1, 1, dk, dv), 2.5)
    out, fin = oracle.prefill(k, k, v, np.zeros((3, 1, dk)), np.ones((3, 1)), [0, 3], 1.0, s0)
    expect = np.full((dk, dv), 2.5)
    for t, c in enumerate(perm):
        expect[c] = v[t, 0]
    assert np.array_equal(fin[0, 0], expect)


# --------------------------------------------------- chunked form cross-check
@pytest.mark.parametrize("chunk", [1, 8, 16, 32, 64])
def test_chunked_equals_token_plain(chunk):
    """I3: the chunked WY/UT form equals the token recurrence for every chunk length
    (different algorithm: catches inclusive/exclusive prefix, decay order, beta placement)."""
    c = _rand_case([1, 31, 32, 33, 70], H=2, dk=16, dv=12)
    out, fin = _run(c)
    out2, fin2 = chunked_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], 0.25,
                                 c["s0"], chunk=chunk)
    _close(out2, out, 1e-11)
    _close(fin2, fin, 1e-11)


def test_chunked_anchored_equals_token():
    """I3 with the fixed anchor C = 16 lb log2(e) at lb = -5 (chunk 32)."""
    c = _rand_case([40, 64, 7], H=2, dk=16, dv=8, lb=-5.0)
    out, fin = _run(c)
    out2, fin2 = chunked_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], 0.25,
                                 c["s0"], chunk=32, mode="anchored", lower_bound=-5.0)
    _close(out2, out, 1e-11)
    _close(fin2, fin, 1e-11)


def test_chunked_split16_equals_token():
    """I3 with the 16-token split factoring at lb = -8."""
    c = _rand_case([45, 32, 3], H=2, dk=16, dv=8, lb=-8.0)
    out, fin = _run(c)
    out2, fin2 = chunked_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], 0.25,
                                 c["s0"], chunk=32, mode="split16", lower_bound=-8.0)
    _close(out2, out, 1e-11)
    _close(fin2, fin, 1e-11)


# ----------------------------------------------------------------- invariants
def test_split_resume():
    """I5: prefill(T1+T2) == prefill(T2, init=final(T1)), at and off multiples of 32."""
    for split in (32, 37, 1):
        c = _rand_case([90], H=2)
        out, fin = _run(c)
        a = {**c, "cu": np.array([0, split]), **{x: c[x][:split] for x in "qkvg"},
             "beta": c["beta"][:split]}
        out_a, fin_a = _run(a)
        b = {**c, "cu": np.array([0, 90 - split]), **{x: c[x][split:] for x in "qkvg"},
             "beta": c["beta"][split:], "s0": fin_a}
        out_b, fin_b = _run(b)
        _close(np.concatenate([out_a, out_b]), out)
        _close(fin_b, fin)


def test_padding_noop():
    """I6: appending tokens with g = 0 and beta = 0 leaves the final state unchanged."""
    c = _rand_case([37], H=2)
    _, fin = _run(c)
    pad = 11
    p = {**c}
    for x in "qkv":
        p[x] = np.concatenate([c[x], np.random.default_rng(3).standard_normal((pad,) + c[x].shape[1:])])
    p["g"] = np.concatenate([c["g"], np.zeros((pad,) + c["g"].shape[1:])])
    p["beta"] = np.concatenate([c["beta"], np.zeros((pad, 2))])
    p["cu"] = np.array([0, 37 + pad])
    _, fin2 = _run(p)
    _close(fin2, fin)


def test_varlen_equals_separate_calls():
    """I7: one packed call == separate per-sequence calls (cu_seqlens handling)."""
    lens = [3, 0, 40, 17]
    c = _rand_case(lens, H=3)
    out, fin = _run(c)
    for n, L in enumerate(lens):
        t0, t1 = c["cu"][n], c["cu"][n + 1]
        one = {**c, "cu": np.array([0, L]), **{x: c[x][t0:t1] for x in "qkvg"},
               "beta": c["beta"][t0:t1], "s0": c["s0"][n:n + 1]}
        o1, f1 = _run(one)
        _close(o1, out[t0:t1])
        _close(f1, fin[n:n + 1])
    assert np.array_equal(fin[1], c["s0"][1])  # empty sequence: final == initial


def test_linearity_in_state_and_values():
    """I8: for fixed (q, k, g, beta) the map (S0, V) -> (O, S_T) is linear."""
    a = _rand_case([50], H=2, seed=11)
    b = _rand_case([50], H=2, seed=12)
    b.update({x: a[x] for x in ("q", "k", "g", "beta")})
    oa, fa = _run(a)
    ob, fb = _run(b)
    s = {**a, "v": 2.0 * a["v"] - 3.0 * b["v"], "s0": 2.0 * a["s0"] - 3.0 * b["s0"]}
    os_, fs = _run(s)
    _close(os_, 2.0 * oa - 3.0 * ob, 1e-11)
    _close(fs, 2.0 * fa - 3.0 * fb, 1e-11)


def test_value_column_independence():
    """I9: value columns evolve independently (basis of any dv split)."""
    c = _rand_case([45, 20], H=2, dv=12)
    out, fin = _run(c)
    cols = [1, 5, 6, 11]
    sub = {**c, "v": c["v"][:, :, cols], "s0": c["s0"][:, :, :, cols]}
    o2, f2 = _run(sub)
    _close(o2, out[:, :, cols])
    _close(f2, fin[:, :, :, cols])


def test_anchor_exponent_range():
    """I10: with g in [lb, 0] the anchored operand exponents G - C and C - G lie in
    [16 lb log2e, -16 lb log2e]: inside the bf16 normal range (|e| <= 126) for
    lb = -5 (random and adversarial all-lb gates), outside it for lb = -8, where the
    16-token split keeps every exponent within 8|lb|log2e."""
    for lb, g_kind, expect_safe in ((-5.0, "random", True), (-5.0, "all_lb", True),
                                    (-5.0, "zero", True), (-8.0, "random", False),
                                    (-8.0, "all_lb", False)):
        c = _rand_case([64], H=1, dk=8, dv=4, lb=lb)
        if g_kind == "all_lb":
            c["g"] = np.full_like(c["g"], lb)
        elif g_kind == "zero":
            c["g"] = np.zeros_like(c["g"])
        audit = {}
        chunked_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], 0.25, c["s0"],
                        chunk=32, mode="anchored", lower_bound=lb, audit=audit)
        lo, hi = audit["anchored"]
        radius = -anchor_constant(lb)
        assert lo >= -radius - 1e-9 and hi <= radius + 1e-9
        assert (max(abs(lo), abs(hi)) <= 126) == expect_safe, (lb, g_kind, lo, hi)
        if lb == -8.0:
            audit = {}
            chunked_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], 0.25, c["s0"],
                            chunk=32, mode="split16", lower_bound=lb, audit=audit)
            lo, hi = audit["split16_diag"]
            assert max(abs(lo), abs(hi)) <= 8 * 8 * 1.4426950408889634 + 1e-9 < 126
            lo, hi = audit["split16_off"]
            assert hi <= 1e-12  # off-diagonal factors only shrink


def test_decode_equals_prefill_T1():
    """I4: one decode step on pool[slot] == prefill of length 1 from that state;
    negative slots skip their row and zero its output."""
    rng = np.random.default_rng(5)
    rows, H, dk, dv, slots_n = 4, 2, 16, 12, 6
    c = _rand_case([1] * rows, H=H, dk=dk, dv=dv)
    pool = rng.standard_normal((slots_n, H, dk, dv))
    slots = np.array([4, -1, 0, 2])
    out, newpool = oracle.decode(c["q"], c["k"], c["v"], c["g"], c["beta"], pool, slots, 0.25)
    for r, s in enumerate(slots):
        if s < 0:
            assert np.all(out[r] == 0.0)
            continue
        o1, f1 = oracle.prefill(c["q"][r:r + 1], c["k"][r:r + 1], c["v"][r:r + 1],
                                c["g"][r:r + 1], c["beta"][r:r + 1], [0, 1], 0.25,
                                pool[s][None])
        _close(out[r], o1[0])
        _close(newpool[s], f1[0])
    for s in (1, 3, 5):
        assert np.array_equal(newpool[s], pool[s])


def test_oracle_rejects_bad_arguments():
    c = _rand_case([4], H=1, dk=16, dv=12)
    with pytest.raises(ValueError):   # slot 5 outside a 2-slot pool
        oracle.decode(c["q"], c["k"], c["v"], c["g"], c["beta"], np.zeros((2, 1, 16, 12)),
                      [5, 0, 1, -1], 1.0)
    with pytest.raises(ValueError):   # decreasing cu_seqlens
        oracle.prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], np.array([0, 3, 2, 4]), 1.0,
                       None)


def test_snapshots_equal_truncated_prefills():
    """State snapshots every I tokens equal the final states of independent prefills of
    the first j*I tokens of each sequence (and the last one equals the final state when
    the length is a multiple of I)."""
    from kimi_delta_attention_prefill_amd.inputs import make_prefill_case
    case = make_prefill_case([130, 64, 40, 96], 2, -5.0, 0.02, seed=31, name="snapshots")
    I = 32
    out, fin, snaps = oracle.prefill(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens,
                                     case.scale, case.initial_state, snapshot_every=I)
    cu = case.cu_seqlens.long().tolist()
    for n in range(case.num_seqs):
        L = cu[n + 1] - cu[n]
        assert snaps[n].shape[0] == L // I
        for j in range(1, L // I + 1):
            sl = slice(cu[n], cu[n] + j * I)
            _, f = oracle.prefill(case.q[sl], case.k[sl], case.v[sl], case.g[sl], case.beta[sl],
                                  np.array([0, j * I]), case.scale, case.initial_state[n:n + 1])
            assert np.array_equal(snaps[n][j - 1], f[0])
        if L % I == 0 and L > 0:
            assert np.array_equal(snaps[n][-1], fin[n])


# ---------------------------------------------------------------- front-end
from oracle import frontend as fe  # noqa: E402


def test_frontend_sigmoid_softplus_closed_forms():
    # sigmoid(0) = 1/2; softplus(0) = ln 2; exact asymptotes far from 0
    assert fe.sigmoid(0.0) == 0.5
    assert fe.softplus(0.0) == math.log(2.0)
    assert fe.softplus(60.0) == 60.0                        # log(1 + e^60) = 60 + O(e^-60)
    assert fe.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-15)
    with np.errstate(over="raise", invalid="raise"):             # no overflow either way
        assert fe.sigmoid(-700.0) == pytest.approx(math.exp(-700.0), rel=1e-15)
        assert fe.sigmoid(-800.0) == 0.0 and fe.sigmoid(800.0) == 1.0
        assert fe.softplus(800.0) == 800.0 and fe.softplus(-800.0) == 0.0
    # sigmoid(x) + sigmoid(-x) = 1 and softplus(x) - softplus(-x) = x, both signs
    x = np.linspace(-30.0, 30.0, 241)
    np.testing.assert_allclose(fe.sigmoid(x) + fe.sigmoid(-x), 1.0, rtol=0, atol=4.5e-16)   # 2 ulp
    np.testing.assert_allclose(fe.softplus(x) - fe.softplus(-x), x, rtol=0, atol=1e-13)
    # sigmoid(x) = exp(-softplus(-x)): two independent formulas of the same function
    np.testing.assert_allclose(fe.sigmoid(x), np.exp(-fe.softplus(-x)), rtol=1e-14)
    # the derivative of softplus is sigmoid (central difference)
    h = 1e-6
    np.testing.assert_allclose((fe.softplus(x + h) - fe.softplus(x - h)) / (2 * h), fe.sigmoid(x),
                               rtol=0, atol=1e-8)


def test_frontend_gates():
    a = np.array([-50.0, -1.0, 0.0, 1.0, 50.0])
    # lower-bound gate: in (lb, 0), lb / 2 at a = 0, -> 0 and -> lb at the ends
    g = fe.gate(a, fe.GATE_LOWER_BOUND, -5.0)
    assert g[2] == -2.5 and g[0] > -1e-20 and g[-1] == -5.0
    assert np.all(np.diff(g) < 0)
    # softplus gate: -ln 2 at 0, -a for large a, unbounded below
    g = fe.gate(a, fe.GATE_SOFTPLUS)
    assert g[2] == -math.log(2.0) and g[-1] == -50.0 and g[0] < 0.0
    # log mode passes the value through
    np.testing.assert_array_equal(fe.gate(a, fe.GATE_LOG), a)
    with pytest.raises(ValueError):
        fe.gate(a, 7)


def test_frontend_l2_norm_axis_and_eps():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 4, 128)) * np.arange(1, 13).reshape(3, 4, 1)
    y = fe.l2_normalize(x, 0.0)
    # unit length over the 128 channels of every (token, head), direction kept
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-14)
    # eps: squared length s / (s + eps); a zero vector stays zero
    s = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(fe.l2_normalize(x, 1e-2) ** 2, axis=-1), s / (s + 1e-2),
                               rtol=1e-14)
    assert np.all(fe.l2_normalize(np.zeros((2, 128)), 1e-6) == 0.0)
    assert np.all(fe.l2_normalize(np.zeros((2, 128)), 0.0) == 0.0)   # no 0/0
    # a basis vector scaled by c normalises to the basis vector exactly
    e = np.zeros(128)
    e[17] = 3.0
    np.testing.assert_array_equal(fe.l2_normalize(e, 0.0), np.eye(128)[17])


def test_frontend_apply_composes():
    rng = np.random.default_rng(6)
    q, k, a = (rng.standard_normal((5, 2, 128)) for _ in range(3))
    b = rng.standard_normal((5, 2))
    q1, k1, g1, b1 = fe.apply(q, k, a, b, gate_mode=fe.GATE_SOFTPLUS, beta_logits=True,
                              normalize_qk=True, norm_eps=1e-6)
    np.testing.assert_allclose(np.linalg.norm(q1, axis=-1), 1.0, atol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(k1, axis=-1), 1.0, atol=1e-6)
    assert np.all(g1 < 0) and np.all((b1 > 0) & (b1 < 1))
    # identity settings change nothing
    q2, k2, g2, b2 = fe.apply(q, k, a, b)
    for u, w in ((q2, q), (k2, k), (g2, a), (b2, b)):
        np.testing.assert_array_equal(u, w)
