"""GPU tests of the device-side precondition checks (kda_check_prefill_inputs,
kda_check_slots): valid inputs raise no flag, and each planted violation --
made on the CPU before the inputs are copied to the device -- raises its own
flag and no other."""
import dataclasses
import sys

import pytest
import torch

import kimi_delta_attention_prefill_amd as kda
from kimi_delta_attention_prefill_amd.inputs import make_decode_case, make_prefill_case

pytestmark = pytest.mark.gpu

NONE = {"cu_seqlens": False, "gate_range": False, "beta_range": False, "qkv_finite": False,
        "gate_steep": False}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kda.load()
    return torch.device("cuda:0")


def _check(case, dev, lower_bound=None):
    print(f"[gpu] check_prefill_inputs {case.name} T={case.total_tokens}", flush=True)
    sys.stdout.flush()
    to = lambda t: t.to(dev)
    return kda.check_prefill_inputs(to(case.q), to(case.k), to(case.v), to(case.g),
                                    to(case.beta), to(case.cu_seqlens),
                                    lower_bound=case.lower_bound if lower_bound is None
                                    else lower_bound)


def _base():
    return make_prefill_case([70, 0, 33, 5], 2, -5.0, 0.02, seed=77, name="check")


def test_valid_inputs_raise_nothing(dev):
    assert _check(_base(), dev) == NONE
    assert _check(_base(), dev, lower_bound=float("-inf")) == NONE


def test_each_violation_raises_its_flag(dev):
    c = _base()
    cu = c.cu_seqlens.clone()
    a, b = int(cu[2]), int(cu[3])
    cu[2], cu[3] = b, a                                 # not monotone: 0, 70, 103, 70, 108
    assert _check(dataclasses.replace(c, cu_seqlens=cu, name="cu"), dev) == dict(NONE, cu_seqlens=True)
    cu = c.cu_seqlens.clone()
    cu[-1] -= 1                                         # last offset != total tokens
    assert _check(dataclasses.replace(c, cu_seqlens=cu, name="cu_end"), dev) == dict(NONE, cu_seqlens=True)
    g = c.g.clone()
    g[40, 1, 77] = -5.5                                 # below the bound
    assert _check(dataclasses.replace(c, g=g, name="g_low"), dev) == dict(NONE, gate_range=True)
    # with no bound only a positive or NaN gate is out of range
    assert _check(dataclasses.replace(c, g=g, name="g_low_unbounded"), dev,
                  lower_bound=float("-inf")) == NONE
    g = c.g.clone()
    g[0, 0, 0] = 0.25                                   # a growing channel
    assert _check(dataclasses.replace(c, g=g, name="g_pos"), dev) == dict(NONE, gate_range=True)
    b = c.beta.clone()
    b[107, 1] = 1.5
    assert _check(dataclasses.replace(c, beta=b, name="beta"), dev) == dict(NONE, beta_range=True)
    v = c.v.clone()
    v[3, 0, 5] = float("nan")
    assert _check(dataclasses.replace(c, v=v, name="v_nan"), dev) == dict(NONE, qkv_finite=True)
    q = c.q.clone()
    q[100, 1, 127] = float("inf")
    assert _check(dataclasses.replace(c, q=q, name="q_inf"), dev) == dict(NONE, qkv_finite=True)


def test_steep_quarter_flag(dev):
    """KDA_CHECK_GATE_STEEP: a gate falling by more than 160.8 nats within an
    8-token quarter of a chunk (tokens 8-15 of the first sequence, 7 x -30)
    is flagged; the same fall split by a sequence boundary is not."""
    c = _base()
    g = c.g.clone()
    g[9:16, 1, 40] = -30.0                              # quarter 8-15 of sequence 0: 210 nats
    assert _check(dataclasses.replace(c, g=g, name="steep"), dev,
                  lower_bound=float("-inf")) == dict(NONE, gate_steep=True)
    g = c.g.clone()
    g[66:74, 0, 3] = -30.0                              # 64-69 in sequence 0, 70-73 in sequence 2
    assert _check(dataclasses.replace(c, g=g, name="steep_split"), dev,
                  lower_bound=float("-inf")) == NONE
    g = c.g.clone()
    g[9:16, 1, 40] = -22.875                            # 7 x 22.875 = 160.1 nats: within the limit
    assert _check(dataclasses.replace(c, g=g, name="steep_edge"), dev,
                  lower_bound=float("-inf")) == NONE


def test_slot_uniqueness(dev):
    d = make_decode_case(300, 8, 4096, with_pool=False)
    slots = d.slots.clone()
    assert not kda.check_slots(slots.to(dev), 4096)
    slots[250] = -1                                     # skipped rows may repeat
    slots[251] = -1
    slots[252] = 5000                                   # out of range: skipped
    assert not kda.check_slots(slots.to(dev), 4096)
    slots[299] = slots[17]
    assert kda.check_slots(slots.to(dev), 4096)
    assert not kda.check_slots(torch.empty(0, dtype=torch.int32, device=dev), 16)
