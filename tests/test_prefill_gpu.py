"""GPU parity of kda_prefill against the FP64 oracle (through the C ABI).

Small cases are compared element by element in full; the full-size
workloads run exactly as the benchmark launches them and are compared on
sampled (sequence, head) units, which the oracle computes independently.
"""
import sys

import numpy as np
import pytest
import torch

import kimi_delta_attention_prefill_amd as kda
import oracle
from kimi_delta_attention_prefill_amd.inputs import make_prefill_case, prefill_config
from _checks import check_out, check_state

pytestmark = pytest.mark.gpu

ROUTES = [kda.ROUTE_SERIAL, kda.ROUTE_CHUNK, kda.ROUTE_SPLIT, kda.ROUTE_STREAM]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kda.load()  # the HIP library must be present on a GPU host
    return torch.device("cuda:0")


def run_gpu(case, route, dev, with_state=True, final=True, out=None, final_state=None):
    to = lambda t: None if t is None else t.to(dev)
    _say(f"[gpu] prefill {case.name or 'case'} route={route} N={case.num_seqs} "
         f"T={case.total_tokens} H={case.num_heads} lb={case.lower_bound}")
    kda.set_prefill_route(route)
    try:
        o, f = kda.prefill(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                           to(case.cu_seqlens), scale=case.scale, lower_bound=case.lower_bound,
                           initial_state=to(case.initial_state) if with_state else None,
                           final_state=final_state if final_state is not None else final,
                           out=out)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    return o, f


def sub_inputs(case, seqs=None, heads=None):
    """Inputs of the chosen sequences and heads, as the oracle takes them."""
    cu = case.cu_seqlens.long().tolist()
    seqs = list(range(case.num_seqs)) if seqs is None else list(seqs)
    heads = list(range(case.num_heads)) if heads is None else list(heads)
    idx = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]).astype(np.int64)
    lens = [cu[n + 1] - cu[n] for n in seqs]
    sub_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    pick = lambda t: t[idx][:, heads]
    s0 = None
    if case.initial_state is not None:
        s0 = case.initial_state[seqs][:, heads]
    return dict(q=pick(case.q), k=pick(case.k), v=pick(case.v), g=pick(case.g),
                beta=case.beta[idx][:, heads], cu=sub_cu, s0=s0, idx=idx, seqs=seqs, heads=heads)


def run_oracle(case, seqs=None, heads=None):
    s = sub_inputs(case, seqs, heads)
    out, fin = oracle.prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu"], case.scale,
                              s["s0"])
    return out, fin, s


def compare(case, o_gpu, f_gpu, seqs=None, heads=None):
    ref_o, ref_f, s = run_oracle(case, seqs, heads)
    g_o = o_gpu.cpu()[torch.as_tensor(s["idx"])][:, s["heads"]]
    r1 = check_out(g_o, ref_o)
    r2 = None
    if f_gpu is not None:
        g_f = f_gpu.cpu()[s["seqs"]][:, s["heads"]]
        r2 = check_state(g_f, ref_f)
    _say(f"   out {r1}  state {r2}")
    return r1, r2


@pytest.mark.parametrize("route", ROUTES)
def test_config0_full(dev, route):
    case = prefill_config(0)
    o, f = run_gpu(case, route, dev)
    compare(case, o, f)


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("lb", [-5.0, -8.0, -1.0])
def test_ragged_lengths(dev, route, lb):
    """Lengths 0, 1 and around chunk multiples, ring wraps (>= 3 chunks), a ragged tail."""
    case = make_prefill_case([1, 31, 32, 33, 95, 0, 64, 7, 200], 3, lb, 0.02, seed=99,
                             name=f"ragged_lb{lb}")
    o, f = run_gpu(case, route, dev)
    compare(case, o, f)


@pytest.mark.parametrize("lengths,route", [([96], kda.ROUTE_CHUNK), ([97], kda.ROUTE_SPLIT),
                                            ([5, 40, 51], kda.ROUTE_CHUNK),
                                            ([5, 40, 52], kda.ROUTE_SPLIT)])
def test_auto_route_around_short_batch_limit(dev, lengths, route):
    """The automatic choice on either side of the short-batch limit (96 tokens in the
    batch): the planner's pick, and the output of the call that takes it."""
    case = make_prefill_case(lengths, 2, -5.0, 0.02, seed=41, name=f"auto_{sum(lengths)}")
    assert kda.plan(case.num_seqs, case.total_tokens, 2, -5.0).route == route
    o, f = run_gpu(case, kda.ROUTE_AUTO, dev)
    compare(case, o, f)


@pytest.mark.parametrize("nseq", [256, 257])
def test_many_sequences_fused(dev, nseq):
    """Many short sequences on the fused route.  Up to 256 sequences each
    block takes its sequence in longest-first order (ties broken by index;
    most lengths here are shared by many sequences), above that in index
    order; every sequence's outputs and state must land in its own rows
    either way, zero-length sequences included."""
    rng = np.random.default_rng(1000 + nseq)
    lengths = [int(x) for x in rng.choice([0, 5, 32, 33, 40, 64, 70], size=nseq)]
    case = make_prefill_case(lengths, 2, -5.0, 0.02, seed=nseq, name=f"many{nseq}")
    o, f = run_gpu(case, kda.ROUTE_CHUNK, dev)
    compare(case, o, f)


@pytest.mark.parametrize("route", ROUTES)
def test_config1_full(dev, route):
    case = prefill_config(1)
    o, f = run_gpu(case, route, dev)
    compare(case, o, f)


@pytest.mark.parametrize("route", ROUTES)
def test_config2_sampled_heads(dev, route):
    case = prefill_config(2)
    o, f = run_gpu(case, route, dev)
    compare(case, o, f, heads=[0, 13, 31])


@pytest.mark.parametrize("route", ROUTES)
def test_config3_sampled_units(dev, route):
    case = prefill_config(3)
    o, f = run_gpu(case, route, dev)
    compare(case, o, f, seqs=[0, 3], heads=[0, 37, 63])


@pytest.mark.parametrize("route", ROUTES)
def test_write_guards_and_state_alias(dev, route):
    """Nothing outside out/final_state is written; final_state may alias initial_state."""
    case = make_prefill_case([70, 33], 2, -5.0, 0.02, seed=5, name="guards")
    T, H = case.total_tokens, case.num_heads
    canary = -12345.0
    big = torch.full((T + 2, H, 128), canary, dtype=torch.bfloat16, device=dev)
    out_view = big[1:T + 1]
    sbig = torch.full((case.num_seqs + 2, H, 128, 128), canary, dtype=torch.float32, device=dev)
    sview = sbig[1:case.num_seqs + 1]
    sview.copy_(case.initial_state.to(dev))
    to = lambda t: t.to(dev)
    kda.set_prefill_route(route)
    try:
        kda.prefill(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                    to(case.cu_seqlens), scale=case.scale, lower_bound=case.lower_bound,
                    initial_state=sview, final_state=sview, out=out_view)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    assert torch.all(big[0] == canary) and torch.all(big[T + 1] == canary)
    assert torch.all(sbig[0] == canary) and torch.all(sbig[-1] == canary)
    compare(case, out_view, sview)


@pytest.mark.parametrize("route", ROUTES)
def test_zero_length_and_no_state(dev, route):
    case = make_prefill_case([0, 5, 0], 2, -5.0, 0.02, seed=6, name="zero_len")
    o, f = run_gpu(case, route, dev)
    assert torch.equal(f[0].cpu(), case.initial_state[0])
    assert torch.equal(f[2].cpu(), case.initial_state[2])
    compare(case, o, f)
    # no initial state (zeros) and no final state requested
    case0 = make_prefill_case([40], 2, -5.0, None, seed=7, name="no_state")
    o, f = run_gpu(case0, route, dev, final=False)
    assert f is None
    compare(case0, o, None)


def test_empty_call_is_noop(dev):
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(1, dtype=torch.int32, device=dev)
    out, fin = kda.prefill(z, z, z, z, torch.empty((0, 2), dtype=torch.bfloat16, device=dev), cu,
                           scale=0.1, lower_bound=-5.0, final_state=True)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 128) and fin.shape == (0, 2, 128, 128)


@pytest.mark.parametrize("route", ROUTES)
def test_deterministic(dev, route):
    case = make_prefill_case([300, 45], 4, -5.0, 0.02, seed=8, name="determinism")
    o1, f1 = run_gpu(case, route, dev)
    o2, f2 = run_gpu(case, route, dev)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("route", ROUTES)
def test_stream_and_graph_replay(dev, route):
    """Runs on a non-default stream and inside a captured graph, replayed with eager
    work and synchronisations in between; every replay matches the eager result."""
    case = make_prefill_case([130, 64], 2, -5.0, 0.02, seed=9, name="graph")
    to = lambda t: t.to(dev)
    q, k, v, g, b, cu, s0 = (to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                             to(case.cu_seqlens), to(case.initial_state))
    out = torch.empty((case.total_tokens, 2, 128), dtype=torch.bfloat16, device=dev)
    fin = torch.empty_like(s0)
    kda.set_prefill_route(route)
    try:
        need = kda.workspace_size(case.num_seqs, case.total_tokens, 2)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            kda.prefill(q, k, v, g, b, cu, scale=case.scale, lower_bound=case.lower_bound,
                        initial_state=s0, final_state=fin, out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref_o, ref_f = out.clone(), fin.clone()
        graph = torch.cuda.CUDAGraph()
        out.zero_()
        with torch.cuda.graph(graph):
            kda.prefill(q, k, v, g, b, cu, scale=case.scale, lower_bound=case.lower_bound,
                        initial_state=s0, final_state=fin, out=out, workspace=ws)
        for _ in range(3):
            out.fill_(0)
            fin.fill_(0)
            _ = torch.randn(1000, device=dev).sum()  # unrelated eager work
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(fin, ref_f)
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    compare(case, ref_o, ref_f)


@pytest.mark.parametrize("which", ["config0", "ragged", "config1"])
def test_two_pass_equals_split_route(dev, which):
    """kda_prefill_prepare + kda_prefill_chain reproduce the SPLIT route of
    kda_prefill bit for bit, with the records on a side stream's timeline."""
    if which == "config0":
        case = prefill_config(0)
    elif which == "ragged":
        case = make_prefill_case([1, 31, 32, 33, 95, 0, 64, 7, 200], 3, -8.0, 0.02, seed=99,
                                 name="ragged_two_pass")
    else:
        case = prefill_config(1)
    o_ref, f_ref = run_gpu(case, kda.ROUTE_SPLIT, dev)
    to = lambda t: None if t is None else t.to(dev)
    cu = to(case.cu_seqlens)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rec = kda.prefill_prepare(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta), cu,
                                  lower_bound=case.lower_bound)
        o, f = kda.prefill_chain(rec, cu, case.num_heads, scale=case.scale,
                                 total_tokens=case.total_tokens,
                                 initial_state=to(case.initial_state), final_state=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert rec.numel() >= kda.records_size(case.num_seqs, case.total_tokens, case.num_heads)
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)


@pytest.mark.parametrize("T,H,lb,state", [(3000, 3, -8.0, 0.02), (5003, 1, -5.0, 0.02),
                                          (1500, 2, -1.0, None)])
def test_split_windows(dev, T, H, lb, state):
    """One long sequence on the split route is cut into windows (maps of the inner
    windows, then each window from its composed initial state); ragged tails, split-16
    anchoring and a missing initial state included."""
    plan = kda.plan(1, T, H, lb, 0, kda.ROUTE_SPLIT)
    assert plan.windows >= 3
    case = make_prefill_case([T], H, lb, state, seed=17 + T, name=f"windows_T{T}_H{H}")
    o, f = run_gpu(case, kda.ROUTE_SPLIT, dev)
    compare(case, o, f)


@pytest.mark.parametrize("lengths,H,lb,state", [([3000, 2500], 3, -5.0, 0.02),
                                                ([2000, 4100, 777], 2, -8.0, 0.02),
                                                ([0, 1500, 31, 4000], 2, -5.0, None)])
def test_split_windows_several_sequences(dev, lengths, H, lb, state):
    """A batch of several sequences whose chains fill little of the device:
    every sequence is cut into windows by its own length (ragged tails, a
    sequence shorter than one window, a zero-length one and split-16
    anchoring included)."""
    T = sum(lengths)
    plan = kda.plan(len(lengths), T, H, lb, 0, kda.ROUTE_SPLIT)
    assert plan.windows >= 3, plan
    case = make_prefill_case(lengths, H, lb, state, seed=29 + T, name=f"windows_{len(lengths)}seq_H{H}")
    o, f = run_gpu(case, kda.ROUTE_SPLIT, dev)
    compare(case, o, f)


def test_split_windows_two_long_sequences(dev):
    """2 x 8192 tokens at H = 8 on the automatic route (the split route with
    windows), sampled heads of both sequences against the oracle."""
    case = make_prefill_case([8192, 8192], 8, -5.0, 0.02, seed=31, name="windows_2x8192_H8")
    plan = kda.plan(2, case.total_tokens, 8, -5.0, 0, kda.ROUTE_AUTO)
    assert plan.route == kda.ROUTE_SPLIT and plan.windows >= 3, plan
    o, f = run_gpu(case, kda.ROUTE_AUTO, dev)
    compare(case, o, f, heads=[0, 7])


def test_split_windows_graph_replay(dev):
    case = make_prefill_case([1500], 2, -5.0, 0.02, seed=23, name="windows_graph")
    to = lambda t: t.to(dev)
    q, k, v, g, b, cu, s0 = (to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                             to(case.cu_seqlens), to(case.initial_state))
    out = torch.empty((case.total_tokens, 2, 128), dtype=torch.bfloat16, device=dev)
    fin = torch.empty_like(s0)
    kda.set_prefill_route(kda.ROUTE_SPLIT)
    try:
        assert kda.plan(1, case.total_tokens, 2, -5.0, 0, kda.ROUTE_SPLIT).windows >= 3
        ws = torch.empty(kda.workspace_size(1, case.total_tokens, 2), dtype=torch.uint8, device=dev)
        kda.prefill(q, k, v, g, b, cu, scale=case.scale, lower_bound=case.lower_bound,
                    initial_state=s0, final_state=fin, out=out, workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_f = out.clone(), fin.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            kda.prefill(q, k, v, g, b, cu, scale=case.scale, lower_bound=case.lower_bound,
                        initial_state=s0, final_state=fin, out=out, workspace=ws)
        for _ in range(3):
            out.fill_(0)
            fin.fill_(0)
            _ = torch.randn(1000, device=dev).sum()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(fin, ref_f)
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    compare(case, ref_o, ref_f)


@pytest.mark.parametrize("route", [kda.ROUTE_CHUNK, kda.ROUTE_SPLIT])
def test_offsets_above_2_31_elements(dev, route):
    """64 sequences x 4096 tokens x 64 heads: each bf16 tensor holds 2^31
    elements (4 GiB), so the last sequences' element offsets exceed 2^31.
    Inputs are drawn on the device from a seeded generator (as the workloads'
    recipe: unit q/k, lb sigmoid gates, sigmoid beta); sampled units of the
    first and last sequences are compared with the oracle."""
    N, L, H, lb = 64, 4096, 64, -5.0
    T = N * L
    gen = torch.Generator(device=dev).manual_seed(2031)

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=dev)
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    q, k = unit((T, H, 128)), unit((T, H, 128))
    v = torch.randn((T, H, 128), generator=gen, device=dev).to(torch.bfloat16)
    g = (lb * torch.sigmoid(torch.randn((T, H, 128), generator=gen, device=dev))).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((T, H), generator=gen, device=dev)).to(torch.bfloat16)
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device=dev)
    print(f"[gpu] prefill offsets>2^31 route={route} N={N} T={T} H={H}", flush=True)
    kda.set_prefill_route(route)
    try:
        out, fin = kda.prefill(q, k, v, g, beta, cu, scale=128 ** -0.5, lower_bound=lb,
                               final_state=True)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    for n, heads in ((0, [5]), (N - 1, [0, 63])):
        rows = slice(n * L, (n + 1) * L)
        sub = lambda t: t[rows][:, heads].cpu()
        ref_o, ref_f = oracle.prefill(sub(q), sub(k), sub(v), sub(g), sub(beta), [0, L],
                                      128 ** -0.5, None)
        r1 = check_out(out[rows][:, heads].cpu(), ref_o)
        r2 = check_state(fin[n:n + 1, heads].cpu(), ref_f)
        _say(f"   seq {n} heads {heads}: out {r1}  state {r2}")
    del q, k, v, g, beta, out, fin
    torch.cuda.empty_cache()
