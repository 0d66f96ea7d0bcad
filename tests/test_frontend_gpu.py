"""GPU parity of the input front-end (raw gates, beta logits, q/k L2 norm)
against the FP64 oracle's front-end followed by the oracle step, through the C
ABI (kda_decode_ex).  The oracle applies oracle/frontend.py to the same bf16
raw inputs in double precision, then runs the token recurrence."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import kimi_delta_attention_prefill_amd as kda
import oracle
from oracle import frontend as ofe
from kimi_delta_attention_prefill_amd.inputs import make_decode_pool, make_decode_raw_case
from _checks import check_bf16_state, check_out, check_state

pytestmark = pytest.mark.gpu

H = 8
NUM_SLOTS = 512


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kda.load()
    return torch.device("cuda:0")


FRONTENDS = {
    "log": kda.FrontEnd(),
    "lower_bound": kda.FrontEnd(gate_mode=kda.GATE_LOWER_BOUND, lower_bound=-5.0,
                                beta_logits=True, normalize_qk=True, norm_eps=1e-6),
    "softplus": kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True, normalize_qk=True,
                             norm_eps=1e-6),
    "softplus_eps": kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=False,
                                 normalize_qk=True, norm_eps=4.0),
}


def _f64(t):
    return t.double().numpy()


@pytest.mark.parametrize("name", list(FRONTENDS))
@pytest.mark.parametrize("state", ["f32", "bf16"])
@pytest.mark.parametrize("rows", [3, 300])
def test_decode_frontend(dev, name, state, rows):
    fe = FRONTENDS[name]
    case = make_decode_raw_case(rows, H, NUM_SLOTS, seed=900 + rows)
    beta = case.beta
    if not fe.beta_logits:   # beta must be in [0, 1] when it is used as given
        beta = torch.sigmoid(case.beta.float()).to(torch.bfloat16)
    if fe.gate_mode == kda.GATE_LOG:   # a log-decay must be <= 0
        case.g = (-case.g.float().abs()).to(torch.bfloat16)
    dt = torch.float32 if state == "f32" else torch.bfloat16
    P = make_decode_pool(NUM_SLOTS, H, dt, 0.02, 77).to(dev)
    sl = case.slots.to(dev)
    pre = P[sl.long()].clone()
    _say(f"[gpu] decode_ex {name} {state} rows={rows}")
    to = lambda t: t.to(dev)
    out = kda.decode(to(case.q), to(case.k), to(case.v), to(case.g), to(beta), P, sl,
                     scale=case.scale, frontend=fe)
    torch.cuda.synchronize()
    q, k, g, b = ofe.apply(_f64(case.q), _f64(case.k), _f64(case.g), _f64(beta),
                           gate_mode=fe.gate_mode,
                           lower_bound=fe.lower_bound, beta_logits=fe.beta_logits,
                           normalize_qk=fe.normalize_qk, norm_eps=fe.norm_eps)
    ref_out, ref_post = oracle.decode(q, k, case.v, g, b, pre.cpu(), np.arange(rows), case.scale)
    r1 = check_out(out.cpu(), ref_out)
    post = P[sl.long()].cpu()
    r2 = check_state(post, ref_post) if state == "f32" else check_bf16_state(post, ref_post)
    _say(f"   out {r1} state {r2}")


def test_decode_frontend_default_equals_plain(dev):
    """A default front-end (log gate, beta as given, no norm) is bitwise kda_decode."""
    case = make_decode_raw_case(64, H, NUM_SLOTS, seed=5)
    g = (-case.g.float().abs()).to(torch.bfloat16)
    beta = torch.sigmoid(case.beta.float()).to(torch.bfloat16)
    outs, pools = [], []
    for fe in (None, kda.FrontEnd()):
        P = make_decode_pool(NUM_SLOTS, H, torch.float32, 0.02, 78).to(dev)
        to = lambda t: t.to(dev)
        outs.append(kda.decode(to(case.q), to(case.k), to(case.v), to(g), to(beta), P,
                               to(case.slots), scale=case.scale, frontend=fe))
        pools.append(P)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(pools[0], pools[1])


# ---------------------------------------------------------------- prefill
from kimi_delta_attention_prefill_amd.inputs import make_prefill_case, make_prefill_raw_case  # noqa: E402

ROUTES = {"serial": kda.ROUTE_SERIAL, "chunk": kda.ROUTE_CHUNK, "split": kda.ROUTE_SPLIT,
          "stream": kda.ROUTE_STREAM}
PREFILL_FE = {
    "lower_bound": (kda.FrontEnd(gate_mode=kda.GATE_LOWER_BOUND, lower_bound=-5.0,
                                 beta_logits=True, normalize_qk=True, norm_eps=1e-6), {}),
    "lower_bound_wide": (kda.FrontEnd(gate_mode=kda.GATE_LOWER_BOUND, lower_bound=-9.0,
                                      beta_logits=True, normalize_qk=True, norm_eps=1e-6), {}),
    "softplus": (kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True, normalize_qk=True,
                              norm_eps=1e-6), {}),
    # strong decays: softplus(4 + 2 N(0,1)) ~ 4 per token, ~64 over a 16-token half
    "softplus_strong": (kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True,
                                     normalize_qk=True, norm_eps=1e-6),
                        dict(gate_mean=4.0, gate_std=2.0)),
}


def _run_prefill_case(dev, route, fe, case, pool=False):
    to = lambda t: None if t is None else t.to(dev)
    kda.set_prefill_route(ROUTES[route])
    try:
        if pool:
            N, H = case.cu_seqlens.numel() - 1, case.q.shape[1]
            P = torch.zeros((N + 3, H, 128, 128), dtype=torch.float32, device=dev)
            slots = torch.arange(N, dtype=torch.int32, device=dev) + 2
            if case.initial_state is not None:
                P[2:2 + N] = case.initial_state.to(dev)
            out, _ = kda.prefill_pool(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                                      to(case.cu_seqlens), slots, P, scale=case.scale,
                                      lower_bound=-5.0, frontend=fe)
            torch.cuda.synchronize()
            return out.cpu(), P[2:2 + N].cpu()
        out, fin = kda.prefill(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                               to(case.cu_seqlens), scale=case.scale, lower_bound=-5.0,
                               initial_state=to(case.initial_state), final_state=True, frontend=fe)
        torch.cuda.synchronize()
        return out.cpu(), fin.cpu()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)


def _prefill_oracle(case, fe):
    q, k, g, b = ofe.apply(_f64(case.q), _f64(case.k), _f64(case.g), _f64(case.beta),
                           gate_mode=fe.gate_mode, lower_bound=fe.lower_bound,
                           beta_logits=fe.beta_logits, normalize_qk=fe.normalize_qk,
                           norm_eps=fe.norm_eps)
    return oracle.prefill(q, k, case.v, g, b, case.cu_seqlens, case.scale, case.initial_state)


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("name", list(PREFILL_FE))
def test_prefill_frontend(dev, route, name):
    fe, gen = PREFILL_FE[name]
    case = make_prefill_raw_case([100, 333, 64], 2, seed=70 + len(name), **gen)
    _say(f"[gpu] prefill_ex {route} {name}")
    out, fin = _run_prefill_case(dev, route, fe, case)
    ref_out, ref_fin = _prefill_oracle(case, fe)
    _say(f"   out {check_out(out, ref_out)} state {check_state(fin, ref_fin)}")


@pytest.mark.parametrize("name", ["softplus", "softplus_strong"])
def test_prefill_frontend_windows_and_pool(dev, name):
    """One long sequence on the split route (windows) and the pooled entry point."""
    fe, gen = PREFILL_FE[name]
    case = make_prefill_raw_case([2000], 3, seed=81, **gen)
    assert kda.plan(1, 2000, 3, float("-inf"), 0, kda.ROUTE_SPLIT).windows >= 3
    ref_out, ref_fin = _prefill_oracle(case, fe)
    for pool in (False, True):
        _say(f"[gpu] prefill_ex windows {name} pool={pool}")
        out, fin = _run_prefill_case(dev, "split", fe, case, pool=pool)
        _say(f"   out {check_out(out, ref_out)} state {check_state(fin, ref_fin)}")


@pytest.mark.parametrize("route", list(ROUTES))
def test_prefill_unbounded_log_gate(dev, route):
    """kda_prefill with lower_bound = -inf: the gate tensor is the log-decay
    itself, unbounded below (data-dependent anchors on the chunk routes)."""
    case = make_prefill_raw_case([300, 45], 2, seed=91, gate_mean=3.0, gate_std=2.0, qk_std=1.0)
    g = -torch.nn.functional.softplus(case.g.float())     # generator-side draw: log-decay <= 0
    case.g = g.to(torch.bfloat16)
    q = case.q.float()
    case.q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    k = case.k.float()
    case.k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    case.beta = torch.sigmoid(case.beta.float()).to(torch.bfloat16)
    to = lambda t: None if t is None else t.to(dev)
    kda.set_prefill_route(ROUTES[route])
    try:
        out, fin = kda.prefill(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                               to(case.cu_seqlens), scale=case.scale, lower_bound=float("-inf"),
                               initial_state=to(case.initial_state), final_state=True)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    ref_out, ref_fin = oracle.prefill(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens,
                                      case.scale, case.initial_state)
    _say(f"[gpu] prefill lb=-inf {route}: out {check_out(out.cpu(), ref_out)} "
         f"state {check_state(fin.cpu(), ref_fin)}")


def _steep_case(seed, lengths, H, steep_channels=6, mean=14.0):
    """Unbounded softplus gates whose chosen channels fall by ~14 nats per
    token (~210 over a 16-token half, beyond a single anchor's 2^248, ~98 per
    8-token quarter), the rest as usual; q, k unit, beta from N(0,1) logits."""
    case = make_prefill_raw_case(lengths, H, seed=seed, qk_std=1.0)
    gen = torch.Generator().manual_seed(seed + 1)
    a = case.g.float()
    ch = torch.randperm(128, generator=gen)[:steep_channels]
    a[:, :, ch] = mean + torch.randn(a.shape[0], H, steep_channels, generator=gen)
    case.g = a.to(torch.bfloat16)
    q = case.q.float()
    case.q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    k = case.k.float()
    case.k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    return case


@pytest.mark.parametrize("route", list(ROUTES))
def test_prefill_steep_unbounded_gates(dev, route):
    """Softplus gates above 200 nats per 16-token half on a few channels, as
    the log-decay (lower_bound = -inf) and through the front-end's softplus
    gate: the chunk routes form those halves' products per 8-token quarter."""
    case = _steep_case(97, [300, 77], 2)
    fe = kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True)
    _say(f"[gpu] prefill steep softplus (front-end) {route}")
    out, fin = _run_prefill_case(dev, route, fe, case)
    ref_out, ref_fin = _prefill_oracle(case, fe)
    _say(f"   out {check_out(out, ref_out)} state {check_state(fin, ref_fin)}")
    # the same gates as a plain log-decay
    g = -torch.nn.functional.softplus(case.g.float())
    plain = dataclasses.replace(case, g=g.to(torch.bfloat16),
                                beta=torch.sigmoid(case.beta.float()).to(torch.bfloat16))
    to = lambda t: None if t is None else t.to(dev)
    kda.set_prefill_route(ROUTES[route])
    try:
        out, fin = kda.prefill(to(plain.q), to(plain.k), to(plain.v), to(plain.g), to(plain.beta),
                               to(plain.cu_seqlens), scale=plain.scale, lower_bound=float("-inf"),
                               initial_state=to(plain.initial_state), final_state=True)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    ref_out, ref_fin = oracle.prefill(plain.q, plain.k, plain.v, plain.g, plain.beta,
                                      plain.cu_seqlens, plain.scale, plain.initial_state)
    _say(f"[gpu] prefill steep lb=-inf {route}: out {check_out(out.cpu(), ref_out)} "
         f"state {check_state(fin.cpu(), ref_fin)}")


def test_prefill_steep_gates_windows_and_pool(dev):
    """Steep softplus gates on one long sequence: the split route with windows
    and the pooled entry point."""
    fe = kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True, normalize_qk=True, norm_eps=1e-6)
    case = _steep_case(99, [2000], 3)
    assert kda.plan(1, 2000, 3, float("-inf"), 0, kda.ROUTE_SPLIT).windows >= 3
    ref_out, ref_fin = _prefill_oracle(case, fe)
    for pool in (False, True):
        _say(f"[gpu] prefill steep windows pool={pool}")
        out, fin = _run_prefill_case(dev, "split", fe, case, pool=pool)
        _say(f"   out {check_out(out, ref_out)} state {check_state(fin, ref_fin)}")


@pytest.mark.parametrize("route", list(ROUTES))
def test_prefill_wide_bound_takes_data_anchors(dev, route):
    """A bound below -10.9 (here -20: g = -20 sigmoid(a), halves falling by up
    to ~300 nats) leaves the 16-token anchors' range; the plan takes the
    data-dependent anchors and the steep halves' quarter products."""
    assert kda.plan(1, 4096, 2, -20.0, 0, kda.ROUTE_CHUNK).anchor_mode == kda.ANCHOR_DATA
    assert kda.plan(1, 4096, 2, -10.0, 0, kda.ROUTE_CHUNK).anchor_mode == kda.ANCHOR_SPLIT16
    case = make_prefill_case([200, 90], 2, -20.0, 0.02, seed=101, name="lb-20")
    out, fin = _run_lb(dev, route, case)
    ref_out, ref_fin = oracle.prefill(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens,
                                      case.scale, case.initial_state)
    _say(f"[gpu] prefill lb=-20 {route}: out {check_out(out.cpu(), ref_out)} "
         f"state {check_state(fin.cpu(), ref_fin)}")


def _run_lb(dev, route, case):
    to = lambda t: None if t is None else t.to(dev)
    kda.set_prefill_route(ROUTES[route])
    try:
        out, fin = kda.prefill(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                               to(case.cu_seqlens), scale=case.scale, lower_bound=case.lower_bound,
                               initial_state=to(case.initial_state), final_state=True)
        torch.cuda.synchronize()
        return out, fin
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
