"""kda_prefill_noalloc (the allocation-free prefill) against kda_prefill.

Both run the same kernels on the same inputs, so the outputs and final
states must agree bit for bit (the floating-point parity of kda_prefill
itself against the oracle is covered by the other prefill tests; here one
sampled head is still checked against the oracle).  Two calls in a row, the
second on a smaller problem, so the second runs on the scratch the first
left behind.  Both take the split route, whose workspace is the scratch.
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


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kda.load()
    kda.set_prefill_route(kda.ROUTE_AUTO)
    return torch.device("cuda:0")


def _inputs(case, dev):
    to = lambda t: None if t is None else t.to(dev)
    return dict(q=to(case.q), k=to(case.k), v=to(case.v), g=to(case.g), beta=to(case.beta),
                cu=to(case.cu_seqlens), s0=to(case.initial_state))


def _both(case, dev):
    x = _inputs(case, dev)
    p = kda.plan(case.num_seqs, case.total_tokens, case.num_heads, case.lower_bound)
    assert p.route == kda.ROUTE_SPLIT, p
    need = kda.workspace_size(case.num_seqs, case.total_tokens, case.num_heads)
    assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES
    _say(f"[gpu] noalloc {case.name or 'case'} N={case.num_seqs} T={case.total_tokens} "
         f"H={case.num_heads} windows={p.windows} workspace={need}")
    o_ref, f_ref = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"],
                               scale=case.scale, lower_bound=case.lower_bound,
                               initial_state=x["s0"], final_state=True)
    o_na, f_na = kda.prefill_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"],
                                     scale=case.scale, lower_bound=case.lower_bound,
                                     initial_state=x["s0"], final_state=True)
    torch.cuda.synchronize()
    return o_ref, f_ref, o_na, f_na


def _oracle_head(case, o_gpu, f_gpu, h):
    cu = case.cu_seqlens.long().tolist()
    s0 = None if case.initial_state is None else case.initial_state[:, [h]]
    ro, rf = oracle.prefill(case.q[:, [h]], case.k[:, [h]], case.v[:, [h]], case.g[:, [h]],
                            case.beta[:, [h]], np.asarray(cu, dtype=np.int64), case.scale, s0)
    check_out(o_gpu.cpu()[:, [h]], ro)
    check_state(f_gpu.cpu()[:, [h]], rf)


def test_noalloc_matches_prefill_two_calls(dev):
    big = prefill_config(1)                                  # 1 x 8192 tokens, H = 8
    small = make_prefill_case([3001], 4, -8.0, init_std=0.02, seed=20299, name="T3001_H4_lb-8")
    for case in (big, small):
        o_ref, f_ref, o_na, f_na = _both(case, dev)
        assert torch.equal(o_na, o_ref), f"{case.name}: outputs differ from kda_prefill"
        assert torch.equal(f_na, f_ref), f"{case.name}: final states differ from kda_prefill"
        _oracle_head(case, o_na, f_na, h=case.num_heads - 1)


def test_noalloc_rejects_oversized_problem(dev):
    # 1 x 2^20 tokens at H = 8 would need gigabytes of chunk records: refused
    # on the host, nothing enqueued (no tensor is read).
    T, H = 1 << 20, 8
    assert kda.workspace_size(1, T, H) > kda.NOALLOC_SCRATCH_BYTES
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    dummy = torch.empty(16, dtype=torch.bfloat16, device=dev)
    lib = kda.load()
    p = dummy.data_ptr()
    rc = lib.kda_prefill_noalloc(p, p, p, p, p, cu.data_ptr(), 1, T, H, 128, 128, 0.088, -5.0,
                                 None, None, p, None)
    assert rc == -3, rc
    assert "static scratch" in kda.last_error()
