"""GPU parity of kda_decode against the FP64 oracle (through the C ABI).

The pool has 4096 slots x 8 heads (2 GiB in FP32).  For each row count the
touched slots are gathered before the step; the oracle runs the step on
those (exact: rows are independent), and the GPU pool is compared on the
touched slots after the step.  Untouched slots must be bitwise unchanged.
"""
import sys

import numpy as np
import pytest
import torch

import kimi_delta_attention_prefill_amd as kda
import oracle
from kimi_delta_attention_prefill_amd.inputs import make_decode_case, make_decode_pool
from _checks import check_bf16_state, check_out, check_state

pytestmark = pytest.mark.gpu

NUM_SLOTS = 4096
H = 8
ROWS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096]
MAX_ORACLE_ROWS = 384


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kda.load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module", params=["f32", "bf16"])
def pool(request, dev):
    dt = torch.float32 if request.param == "f32" else torch.bfloat16
    return request.param, make_decode_pool(NUM_SLOTS, H, dt, 0.02, 4242).to(dev)


def _step(case, pool_t, dev, slots=None):
    to = lambda t: t.to(dev)
    sl = to(case.slots if slots is None else slots)
    out = kda.decode(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta), pool_t, sl,
                     scale=case.scale)
    torch.cuda.synchronize()
    return out


def _oracle_rows(case, pre_states, rows_idx):
    """Oracle step for the chosen rows; pre_states[i] is the state of row rows_idx[i]."""
    sel = torch.as_tensor(rows_idx)
    return oracle.decode(case.q[sel], case.k[sel], case.v[sel], case.g[sel], case.beta[sel],
                         pre_states, np.arange(len(rows_idx)), case.scale)


@pytest.mark.parametrize("rows", ROWS)
def test_decode_rows(dev, pool, rows):
    tag, P = pool
    case = make_decode_case(rows, H, NUM_SLOTS, seed=1000 + rows, with_pool=False)
    _say(f"[gpu] decode {tag} rows={rows}")
    slots_d = case.slots.to(dev).long()
    pre = P[slots_d].clone()
    check_untouched = rows in (1, 64, 4096 if tag == "bf16" else 1024)
    before = P.clone() if check_untouched else None
    out = _step(case, P, dev)
    post = P[slots_d]
    rng = np.random.default_rng(rows)
    rows_idx = np.arange(rows) if rows <= MAX_ORACLE_ROWS else np.sort(
        rng.choice(rows, MAX_ORACLE_ROWS, replace=False))
    ref_out, ref_post = _oracle_rows(case, pre[torch.as_tensor(rows_idx, device=dev)].cpu(),
                                     rows_idx)
    r1 = check_out(out.cpu()[torch.as_tensor(rows_idx)], ref_out)
    g_post = post[torch.as_tensor(rows_idx, device=dev)].cpu()
    r2 = check_state(g_post, ref_post) if tag == "f32" else check_bf16_state(g_post, ref_post)
    _say(f"   out {r1} state {r2}")
    if check_untouched:
        mask = torch.ones(NUM_SLOTS, dtype=torch.bool, device=dev)
        mask[slots_d] = False
        assert torch.equal(P[mask], before[mask]), "untouched slots changed"
        del before


@pytest.mark.parametrize("rows", [6, 1200])
def test_decode_negative_and_out_of_range_slots(dev, pool, rows):
    """Skipped rows (negative or out-of-range slot): zero output, pool untouched.
    At 1200 rows x H=8 both pools take the many-row shape (the token stream
    with one token per row), at 6 rows the decode blocks."""
    tag, P = pool
    case = make_decode_case(rows, H, NUM_SLOTS, seed=77 + rows, with_pool=False)
    slots = case.slots.clone()
    slots[1] = -1
    slots[4] = NUM_SLOTS + 5   # out of range: treated as a skipped row
    slots[rows - 1] = -7
    dead = {1, 4, rows - 1}
    live = [i for i in range(rows) if i not in dead]
    if len(live) > MAX_ORACLE_ROWS:
        live = sorted(np.random.default_rng(rows).choice(live, MAX_ORACLE_ROWS, replace=False))
    slots_d = slots.to(dev).long()
    pre = P[slots_d[live]].clone()
    before = P.clone()
    out = _step(case, P, dev, slots=slots)
    for r in dead:
        assert torch.all(out[r] == 0), f"skipped row {r} has a nonzero output"
    ref_out, ref_post = _oracle_rows(case, pre.cpu(), np.array(live))
    check_out(out.cpu()[live], ref_out)
    post = P[slots_d[live]].cpu()
    (check_state if tag == "f32" else check_bf16_state)(post, ref_post)
    valid = slots_d[[i for i in range(rows) if i not in dead]]
    mask = torch.ones(NUM_SLOTS, dtype=torch.bool, device=dev)
    mask[valid] = False
    assert torch.equal(P[mask], before[mask])
    del before


def test_decode_matches_prefill_T1(dev):
    """One decode step from a state == prefill of length 1 from the same state (FP32)."""
    rows = 5
    case = make_decode_case(rows, H, 16, seed=31)
    P = case.pool.to(dev)
    init = P[case.slots.to(dev).long()].clone()           # [rows, H, 128, 128]
    out_d = _step(case, P, dev)
    post = P[case.slots.to(dev).long()]
    to = lambda t: t.to(dev)
    cu = torch.arange(rows + 1, dtype=torch.int32, device=dev)
    kda.set_prefill_route(kda.ROUTE_SERIAL)
    try:
        o_p, f_p = kda.prefill(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta), cu,
                               scale=case.scale, lower_bound=-30.0, initial_state=init,
                               final_state=True)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    check_out(out_d.cpu(), o_p.cpu().double(), tol=1e-3)
    check_state(post.cpu(), f_p.cpu().double(), tol=1e-4)
