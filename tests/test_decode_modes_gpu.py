"""GPU tests of the decode (and pooled prefill) serving modes, through the C ABI.

The serving cases the fused-decode PR lists ("Kimi K3 TP12 H=8 fused KDA
decode", flashinfer PR #5551, its GPU test notes): a 16,384-slot pool whose
offsets need 64 bits, with only the live slots randomised; page and padded
pool layouts; batches padded with null slots; caller-owned outputs with
prefix/suffix write guards; graph replay.  Readings: the "page" layout is the
dense [num_slots, H, 128, 128] pool, the "padded" layout puts the slots at a
larger stride (here one layer's view of a [num_slots, layers, H, 128, 128]
pool), and a padded batch carries null (-1) slots after its live rows.

Every result is checked against the FP64 oracle on the gathered live states
(rows are independent, so this is exact), and every slot the step must not
touch is checked bitwise.
"""
import sys

import numpy as np
import pytest
import torch

import kimi_delta_attention_prefill_amd as kda
import oracle
from kimi_delta_attention_prefill_amd.inputs import make_decode_case, make_prefill_case
from _checks import check_bf16_state, check_out, check_state

pytestmark = pytest.mark.gpu

H = 8


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kda.load()
    return torch.device("cuda:0")


def _check_rows(case, out, pre, post, live_rows, bf16):
    """Oracle step on the live rows from their pre-step states; compare."""
    sel = torch.as_tensor(live_rows)
    ref_out, ref_post = oracle.decode(case.q[sel], case.k[sel], case.v[sel], case.g[sel],
                                      case.beta[sel], pre, np.arange(len(live_rows)), case.scale)
    r1 = check_out(out.cpu()[sel], ref_out)
    r2 = (check_bf16_state if bf16 else check_state)(post, ref_post)
    return r1, r2


def _live_states(num, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return (0.02 * torch.randn((num, H, 128, 128), generator=g)).to(dtype)


LARGE = [  # (state dtype, layers of the padded view; 1 = dense page layout)
    (torch.float32, 1),    # 8 GiB, byte offsets up to 2^33
    (torch.bfloat16, 1),   # 4 GiB
    (torch.bfloat16, 2),   # 8 GiB, layer 1's view: element offsets above 2^31
]


@pytest.mark.parametrize("dtype,layers", LARGE, ids=["f32", "bf16", "bf16_padded"])
def test_decode_16384_slot_pool(dev, dtype, layers):
    num_slots, rows = 16384, 300
    case = make_decode_case(rows, H, num_slots, seed=5151, with_pool=False)
    slots = case.slots.clone()
    top = [num_slots - 1, num_slots - 2, num_slots // 2]
    for i, s in enumerate(top):   # the largest offsets are always exercised
        hit = (slots == s).nonzero()
        if hit.numel():
            slots[hit[0, 0]] = slots[i]
        slots[i] = s
    assert torch.unique(slots).numel() == rows
    _say(f"[gpu] decode 16384-slot pool dtype={dtype} layers={layers} rows={rows}")
    base = torch.zeros((num_slots, layers, H, 128, 128), dtype=dtype, device=dev)
    pool = base[:, layers - 1]
    live = slots.to(dev).long()
    pool[live] = _live_states(rows, dtype, 5152).to(dev)   # only the live slots are random
    pre = pool[live].cpu()
    out = kda.decode(case.q.to(dev), case.k.to(dev), case.v.to(dev), case.g.to(dev),
                     case.beta.to(dev), pool, slots.to(dev), scale=case.scale)
    torch.cuda.synchronize()
    post = pool[live].cpu()
    r = _check_rows(case, out, pre, post, np.arange(rows), dtype == torch.bfloat16)
    _say(f"   {r}")
    # nothing but the live slots' states (in the viewed layer) is nonzero
    written = base.view(num_slots * layers, -1).ne(0).any(dim=1).view(num_slots, layers)
    expect = torch.zeros_like(written)
    expect[live, layers - 1] = True
    assert torch.equal(written, expect), "a slot or layer outside the live rows was written"
    del base, pool, written
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("rows", [5, 300])
def test_decode_padded_layout_and_batch(dev, dtype, rows):
    """Slots at a padded stride (layer 1 of 3), and a batch padded with null slots."""
    num_slots, layers, pad = 384, 3, 7
    case = make_decode_case(rows + pad, H, num_slots, seed=6161 + rows, with_pool=False)
    slots = case.slots.clone()
    slots[rows:] = -1
    g = torch.Generator().manual_seed(6162)
    base = (0.02 * torch.randn((num_slots, layers, H, 128, 128), generator=g)).to(dtype).to(dev)
    before = base.clone()
    pool = base[:, 1]
    live = slots[:rows].to(dev).long()
    pre = pool[live].cpu()
    _say(f"[gpu] decode padded layout dtype={dtype} rows={rows}+{pad} null")
    out = kda.decode(case.q.to(dev), case.k.to(dev), case.v.to(dev), case.g.to(dev),
                     case.beta.to(dev), pool, slots.to(dev), scale=case.scale)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[rows:]) == 0, "padding rows must give zero output"
    _check_rows(case, out, pre, pool[live].cpu(), np.arange(rows), dtype == torch.bfloat16)
    mask = torch.ones((num_slots, layers), dtype=torch.bool, device=dev)
    mask[live, 1] = False
    assert torch.equal(base[mask], before[mask]), "a state outside the live rows changed"


def test_decode_caller_owned_out_guards(dev):
    rows = 40
    case = make_decode_case(rows, H, 256, seed=7171)
    pool = case.pool.to(dev)
    live = case.slots.to(dev).long()
    pre = pool[live].cpu()
    big = torch.full((rows + 2, H, 128), 7.0, dtype=torch.bfloat16, device=dev)
    out = big[1:-1]
    ret = kda.decode(case.q.to(dev), case.k.to(dev), case.v.to(dev), case.g.to(dev),
                     case.beta.to(dev), pool, case.slots.to(dev), scale=case.scale, out=out)
    torch.cuda.synchronize()
    assert ret.data_ptr() == out.data_ptr()
    assert torch.all(big[0] == 7.0) and torch.all(big[-1] == 7.0), "write outside out"
    _check_rows(case, out, pre, pool[live].cpu(), np.arange(rows), False)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decode_graph_replay(dev, dtype):
    """Three replays of a captured step, eager work between them, each equal
    (bitwise) to the same step run eagerly on a copy of the pool."""
    rows = 96
    case = make_decode_case(rows, H, 512, state_dtype=dtype, seed=8181)
    to = lambda t: t.to(dev)
    q, k, v, g, b, sl = map(to, (case.q, case.k, case.v, case.g, case.beta, case.slots))
    pool = to(case.pool)
    ref_pool = pool.clone()
    out = torch.empty((rows, H, 128), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the binding outside the capture
        kda.decode(q, k, v, g, b, pool.clone(), sl, scale=case.scale, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.decode(q, k, v, g, b, pool, sl, scale=case.scale, out=out)
    _say(f"[gpu] decode graph replay dtype={dtype}")
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        ref_out = kda.decode(q, k, v, g, b, ref_pool, sl, scale=case.scale)
        junk = torch.randn(1 << 20, device=dev).sum()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, ref_out), f"replay {rep}: output differs from the eager step"
        assert torch.equal(pool, ref_pool), f"replay {rep}: pool differs from the eager step"


def test_prefill_pool_graph_replay(dev):
    """kda_prefill_pool captured once (caller-owned out, workspace and
    checkpoints) and replayed from a reset pool: each replay equals the eager
    call bitwise."""
    lengths, Hp, lb = [1500, 45, 300], 4, -5.0
    case = make_prefill_case(lengths, Hp, lb, None, seed=9191)
    N, T = case.num_seqs, case.total_tokens
    to = lambda t: t.to(dev)
    q, k, v, g, b, cu = map(to, (case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens))
    slots = to(torch.tensor([3, -1, 0], dtype=torch.int32))
    gen = torch.Generator().manual_seed(9192)
    pool0 = to((0.02 * torch.randn((5, Hp, 128, 128), generator=gen)).float())
    out = torch.empty((T, Hp, 128), dtype=torch.bfloat16, device=dev)
    ck = torch.zeros((kda.checkpoint_slots(N, T, 64), Hp, 128, 128), device=dev)
    ws = torch.empty(max(kda.workspace_size(N, T, Hp), 1), dtype=torch.uint8, device=dev)
    ref_pool = pool0.clone()
    ref_out, ref_ck = kda.prefill_pool(q, k, v, g, b, cu, slots, ref_pool, scale=case.scale,
                                       lower_bound=lb, checkpoints=True)
    torch.cuda.synchronize()
    pool = pool0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kda.prefill_pool(q, k, v, g, b, cu, slots, pool, scale=case.scale, lower_bound=lb,
                         checkpoints=ck, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.prefill_pool(q, k, v, g, b, cu, slots, pool, scale=case.scale, lower_bound=lb,
                         checkpoints=ck, out=out, workspace=ws)
    _say(f"[gpu] prefill_pool graph replay lengths={lengths} H={Hp}")
    for rep in range(3):
        pool.copy_(pool0)
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, ref_out), f"replay {rep}: output differs"
        assert torch.equal(pool, ref_pool), f"replay {rep}: pool differs"
        assert torch.equal(ck, ref_ck), f"replay {rep}: checkpoints differ"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("route", [kda.ROUTE_SERIAL, kda.ROUTE_CHUNK, kda.ROUTE_SPLIT, kda.ROUTE_STREAM])
def test_prefill_pool_padded_layout(dev, dtype, route):
    """Pooled prefill on layer 1 of a [slots, 3, H, 128, 128] pool: results as
    on a dense pool (checked against the oracle), other layers untouched."""
    lengths, Hp, lb, num_slots = [200, 0, 77, 64], 3, -5.0, 6
    slots = [4, 1, -1, 0]
    case = make_prefill_case(lengths, Hp, lb, None, seed=9393)
    to = lambda t: t.to(dev)
    gen = torch.Generator().manual_seed(9394)
    base = (0.02 * torch.randn((num_slots, 3, Hp, 128, 128), generator=gen)).to(dtype)
    before = to(base.clone())
    base = to(base)
    pool = base[:, 1]
    pre = pool.cpu().double()
    _say(f"[gpu] prefill_pool padded layout dtype={dtype} route={route}")
    kda.set_prefill_route(route)
    try:
        out, _ = kda.prefill_pool(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                                  to(case.cu_seqlens), to(torch.tensor(slots, dtype=torch.int32)),
                                  pool, scale=case.scale, lower_bound=lb)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    s0 = np.stack([pre[s].numpy() if s >= 0 else np.zeros((Hp, 128, 128)) for s in slots])
    ref_o, ref_f = oracle.prefill(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens,
                                  case.scale, s0)
    check_out(out.cpu(), ref_o)
    post = pool.cpu()
    for n, s in enumerate(slots):
        if s >= 0:
            if dtype == torch.bfloat16:
                check_bf16_state(post[s:s + 1], ref_f[n:n + 1], tol=1e-2)
            else:
                check_state(post[s:s + 1], ref_f[n:n + 1])
    mask = torch.ones((num_slots, 3), dtype=torch.bool, device=dev)
    for s in slots:
        if s >= 0:
            mask[s, 1] = False
    assert torch.equal(base[mask], before[mask]), "a state outside the live sequences changed"
