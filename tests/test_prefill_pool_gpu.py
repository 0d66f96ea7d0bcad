"""GPU parity of kda_prefill_pool (states in a slot-indexed FP32 pool, updated in place,
and intermediate-state checkpoints) against the FP64 oracle, on every prefill route."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prefill_amd as kda
import oracle
from kimi_delta_attention_prefill_amd.inputs import make_prefill_case
from _checks import check_bf16_state, check_out, check_state

pytestmark = pytest.mark.gpu

ROUTES = [kda.ROUTE_SERIAL, kda.ROUTE_CHUNK, kda.ROUTE_SPLIT, kda.ROUTE_STREAM]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kda.load()
    return torch.device("cuda:0")


def run_case(dev, route, lengths, H, lb, slots, num_slots, ck_tokens, seed, windows=False,
             bf16_pool=False):
    case = make_prefill_case(lengths, H, lb, None, seed=seed, name=f"pool_{route}")
    N, T = case.num_seqs, case.total_tokens
    g = torch.Generator().manual_seed(seed + 1)
    pool0 = (0.02 * torch.randn((num_slots, H, 128, 128), generator=g)).float()
    if bf16_pool:   # the states the oracle starts from are the bf16 values, read exactly
        pool0 = pool0.to(torch.bfloat16)
    slots_t = torch.tensor(slots, dtype=torch.int32)
    to = lambda t: t.to(dev)
    pool = to(pool0.clone())
    print(f"[gpu] prefill_pool route={route} N={N} T={T} H={H} slots={slots} every={ck_tokens} "
          f"pool={pool0.dtype}", flush=True)
    kda.set_prefill_route(route)
    try:
        if windows:
            assert kda.plan(N, T, H, lb, 0, route).windows >= 3
        out, ck = kda.prefill_pool(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                                   to(case.cu_seqlens), to(slots_t), pool, scale=case.scale,
                                   lower_bound=lb, checkpoints=True, checkpoint_tokens=ck_tokens)
        torch.cuda.synchronize()
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)
    # oracle: gather initial states, run, scatter back
    valid = [0 <= s < num_slots for s in slots]
    s0 = np.stack([pool0[s].double().numpy() if ok else np.zeros((H, 128, 128))
                   for s, ok in zip(slots, valid)])
    ref_o, ref_f, snaps = oracle.prefill(case.q, case.k, case.v, case.g, case.beta,
                                         case.cu_seqlens, case.scale, s0,
                                         snapshot_every=ck_tokens)
    r = check_out(out.cpu(), ref_o)
    pool_cpu = pool.cpu()
    touched = set()
    for n, (s, ok) in enumerate(zip(slots, valid)):
        if ok:
            touched.add(s)
            if bf16_pool:   # the prefill state bound on top of the stored value's bf16 rounding
                check_bf16_state(pool_cpu[s:s + 1], ref_f[n:n + 1], tol=1e-2)
            else:
                check_state(pool_cpu[s:s + 1], ref_f[n:n + 1])
    for s in range(num_slots):
        if s not in touched:
            assert torch.equal(pool_cpu[s], pool0[s]), f"pool slot {s} was modified"
    ck_cpu = ck.cpu()
    cu = case.cu_seqlens.long().tolist()
    used = set()
    for n in range(N):
        for j in range(1, (cu[n + 1] - cu[n]) // ck_tokens + 1):
            slot = n + cu[n] // ck_tokens + j - 1
            assert slot not in used
            used.add(slot)
            check_state(ck_cpu[slot:slot + 1], snaps[n][j - 1][None])
    for slot in range(ck_cpu.shape[0]):
        if slot not in used:
            assert torch.count_nonzero(ck_cpu[slot]) == 0, f"checkpoint slot {slot} written"
    return r


@pytest.mark.parametrize("route", ROUTES)
def test_pool_and_checkpoints(dev, route):
    # a skipped sequence (slot -1), a zero-length one, lengths around the interval
    run_case(dev, route, [130, 64, 0, 200, 33], 3, -5.0, [5, 2, 7, -1, 0], 8, 64, seed=41)


@pytest.mark.parametrize("route", ROUTES)
def test_checkpoints_every_chunk_split16(dev, route):
    run_case(dev, route, [96, 45, 128], 2, -8.0, [1, 0, 3], 4, 32, seed=43)


def test_pool_checkpoints_windows(dev):
    # one long sequence on the windowed split route; checkpoints cross window boundaries
    run_case(dev, kda.ROUTE_SPLIT, [3000], 3, -5.0, [1], 3, 96, seed=47, windows=True)


@pytest.mark.parametrize("route", ROUTES)
def test_bf16_pool(dev, route):
    """A bf16 state pool: states widened on entry, stored back rounded (checkpoints FP32)."""
    run_case(dev, route, [45, 0, 200, 96], 3, -5.0, [4, 1, -1, 6], 8, 64, seed=611,
             bf16_pool=True)


def test_bf16_pool_windows(dev):
    run_case(dev, kda.ROUTE_SPLIT, [2000], 3, -8.0, [2], 4, 96, seed=612, windows=True,
             bf16_pool=True)


def test_many_sequences_fused_pool(dev):
    """40 sequences of shared, varied lengths on the fused route, whose blocks take
    their sequence in longest-first order: every sequence's state must come from
    and return to its own slot, and its checkpoints land in its own rows."""
    rng = np.random.default_rng(613)
    lengths = [int(x) for x in rng.choice([0, 31, 64, 65, 128, 200], size=40)]
    slots = [int(s) for s in rng.permutation(64)[:40]]
    slots[7] = -1                                   # one skipped sequence
    run_case(dev, kda.ROUTE_CHUNK, lengths, 2, -5.0, slots, 64, 64, seed=613)
