"""GPU parity of multi-token decode: T = 2, 4 or 8 new tokens per row, run
through kda_prefill_pool_ex against a 4096-slot state pool at H = 8, with the
input front-end of a model's decode step (softplus gates, beta logits, q/k
L2-normalised).  Each row is a sequence of T tokens whose state lives in the
pool slot the row names (flashinfer PR #5551 "Kimi K3 TP12 H=8 fused KDA
decode", its T > 1 multi-token path); the oracle applies the FP64 front-end
and runs the token recurrence from the same pool states.  At 4096 rows the
oracle checks a sample of rows (rows are independent sequences)."""
import sys

import numpy as np
import pytest
import torch

import kimi_delta_attention_prefill_amd as kda
import oracle
from oracle import frontend as ofe
from kimi_delta_attention_prefill_amd.inputs import make_decode_pool, make_prefill_raw_case
from _checks import check_bf16_state, check_out, check_state

pytestmark = pytest.mark.gpu

H = 8
NUM_SLOTS = 4096
SAMPLE_ROWS = 256
FE = kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True, normalize_qk=True,
                  norm_eps=1e-6)


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
    P = make_decode_pool(NUM_SLOTS, H, dt, 0.02, 4242).to(dev)
    yield request.param, P
    del P
    torch.cuda.empty_cache()


def _f64(t):
    return t.double().numpy()


@pytest.mark.parametrize("rows", [1, 64, 4096])
@pytest.mark.parametrize("tokens", [2, 4, 8])
def test_multitoken_decode(dev, pool, rows, tokens):
    tag, P = pool
    case = make_prefill_raw_case([tokens] * rows, H, init_std=None, seed=7000 + 10 * rows + tokens)
    gen = torch.Generator().manual_seed(7100 + rows + tokens)
    slots = torch.randperm(NUM_SLOTS, generator=gen)[:rows].to(torch.int32)
    sl = slots.to(dev)
    pre = P[sl.long()].clone()
    before = P.clone() if rows < NUM_SLOTS else None
    plan = kda.plan(rows, rows * tokens, H, float("-inf"), 0, kda.ROUTE_AUTO)
    _say(f"[gpu] multitoken decode {tag} rows={rows} T={tokens} plan={plan}")
    to = lambda t: t.to(dev)
    out, _ = kda.prefill_pool(to(case.q), to(case.k), to(case.v), to(case.g), to(case.beta),
                              to(case.cu_seqlens), sl, P, scale=case.scale,
                              lower_bound=float("-inf"), frontend=FE)
    torch.cuda.synchronize()
    post = P[sl.long()].cpu()

    # oracle on all rows, or on a sample of them at 4096 rows
    pick = np.arange(rows) if rows <= SAMPLE_ROWS else np.sort(
        np.random.default_rng(rows + tokens).choice(rows, SAMPLE_ROWS, replace=False))
    tok = (pick[:, None] * tokens + np.arange(tokens)[None, :]).reshape(-1)
    sel = torch.as_tensor(tok)
    q, k, g, b = ofe.apply(_f64(case.q[sel]), _f64(case.k[sel]), _f64(case.g[sel]),
                           _f64(case.beta[sel]), gate_mode=FE.gate_mode,
                           lower_bound=FE.lower_bound, beta_logits=FE.beta_logits,
                           normalize_qk=FE.normalize_qk, norm_eps=FE.norm_eps)
    cu = np.arange(len(pick) + 1, dtype=np.int64) * tokens
    s0 = pre[torch.as_tensor(pick, device=dev)].cpu()
    ref_out, ref_fin = oracle.prefill(q, k, case.v[sel], g, b, cu, case.scale, s0)
    r1 = check_out(out.cpu()[sel], ref_out)
    got = post[torch.as_tensor(pick)]
    r2 = check_state(got, ref_fin) if tag == "f32" else check_bf16_state(got, ref_fin, tol=1e-2)
    _say(f"   out {r1} state {r2}")
    if before is not None:
        mask = torch.ones(NUM_SLOTS, dtype=torch.bool, device=dev)
        mask[sl.long()] = False
        assert torch.equal(P[mask], before[mask]), "untouched slots changed"
        del before
