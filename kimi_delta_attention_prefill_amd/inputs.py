"""Seeded synthetic inputs for KDA prefill and decode.

This module is the only code shared by the GPU path's tests/benchmark and the
FP64 oracle.  It draws random tensors and applies the input recipe (L2
normalisation of q and k, the gate and beta squashing); it contains none of
the recurrence's arithmetic.  Everything is generated on the CPU with
``torch.Generator`` so the same seed gives the same tensors on any host.

Recipe (the workload shapes of the KDA prefill/decode pages; values are
synthetic, there is no dataset):

* q, k ~ N(0, 1) per entry, L2-normalised over the 128 channels of each
  (token, head) in fp32, then rounded to bf16.
* v ~ N(0, 1) -> bf16.
* prefill gate g = lower_bound * sigmoid(a), a ~ N(0, 1), per channel, fp32
  then bf16 (lower_bound is bf16-exact, so g stays in [lower_bound, 0]).
* decode gate g = -softplus(a) = -log1p(exp(a)), a ~ N(0, 1) -> bf16.
* beta = sigmoid(N(0, 1)) per (token, head) -> bf16 (post-sigmoid, in [0, 1]).
* initial states / pool: std * N(0, 1) in fp32 (std = 0.02), or zeros.
* varlen lengths: uniform integers in [min_len, max_len].
* decode slots: the first ``rows`` entries of a random permutation of the
  pool's slots (unique, scattered).

Draw order per case: lengths (varlen only), q, k, v, gate logits, beta
logits, then for prefill the initial state, for decode the slots and then
the pool (last, so a caller can supply its own pool and keep the same rows).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

HEAD_DIM = 128
SCALE = 1.0 / (HEAD_DIM ** 0.5)
BASE_SEED = 20260

__all__ = ["PrefillCase", "DecodeCase", "make_prefill_case", "make_decode_case", "make_decode_pool",
           "prefill_config", "decode_config", "PREFILL_CONFIGS", "SCALE", "HEAD_DIM",
           "BASE_SEED"]


@dataclass
class PrefillCase:
    q: torch.Tensor             # bf16 [T, H, 128]
    k: torch.Tensor             # bf16 [T, H, 128]
    v: torch.Tensor             # bf16 [T, H, 128]
    g: torch.Tensor             # bf16 [T, H, 128]
    beta: torch.Tensor          # bf16 [T, H]
    cu_seqlens: torch.Tensor    # int32 [N + 1]
    initial_state: Optional[torch.Tensor]  # fp32 [N, H, 128, 128] or None (zeros)
    lower_bound: float
    scale: float = SCALE
    seed: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.numel()) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])


@dataclass
class DecodeCase:
    q: torch.Tensor             # bf16 [rows, H, 128]
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor             # bf16 [rows, H, 128]
    beta: torch.Tensor          # bf16 [rows, H]
    pool: Optional[torch.Tensor]  # fp32 or bf16 [num_slots, H, 128, 128]
    slots: torch.Tensor         # int32 [rows]
    scale: float = SCALE
    seed: int = 0
    name: str = ""


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_prefill_case(lengths, num_heads, lower_bound, init_std=None, seed=BASE_SEED,
                      name="", dk=HEAD_DIM, dv=HEAD_DIM) -> PrefillCase:
    """Packed varlen prefill inputs for the given sequence lengths."""
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    H = int(num_heads)
    q = _unit_rows(torch.randn(T, H, dk, generator=gen)).to(torch.bfloat16)
    k = _unit_rows(torch.randn(T, H, dk, generator=gen)).to(torch.bfloat16)
    v = torch.randn(T, H, dv, generator=gen).to(torch.bfloat16)
    lb = float(torch.tensor(lower_bound, dtype=torch.bfloat16).float())
    if lb != float(lower_bound):
        raise ValueError("lower_bound must be exactly representable in bf16")
    g = (lb * torch.sigmoid(torch.randn(T, H, dk, generator=gen))).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn(T, H, generator=gen)).to(torch.bfloat16)
    s0 = None
    if init_std is not None:
        s0 = float(init_std) * torch.randn(len(lengths), H, dk, dv, generator=gen)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return PrefillCase(q, k, v, g, beta, cu, s0, lb, SCALE, int(seed), name,
                       {"lengths": lengths})


def make_prefill_raw_case(lengths, num_heads, init_std=0.02, seed=BASE_SEED + 6, qk_std=3.0,
                          gate_mean=0.0, gate_std=1.0, name="raw") -> PrefillCase:
    """Prefill inputs as a model hands them over before the input front-end:
    q, k ~ qk_std N(0, 1) (not normalised), v ~ N(0, 1), the gate tensor holds
    raw a ~ gate_mean + gate_std N(0, 1), beta holds logits ~ N(0, 1); all
    bf16.  ``lower_bound`` is -inf (the case carries no bound)."""
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    H = int(num_heads)
    q = (float(qk_std) * torch.randn(T, H, HEAD_DIM, generator=gen)).to(torch.bfloat16)
    k = (float(qk_std) * torch.randn(T, H, HEAD_DIM, generator=gen)).to(torch.bfloat16)
    v = torch.randn(T, H, HEAD_DIM, generator=gen).to(torch.bfloat16)
    a = (float(gate_mean) + float(gate_std) * torch.randn(T, H, HEAD_DIM, generator=gen)
         ).to(torch.bfloat16)
    b = torch.randn(T, H, generator=gen).to(torch.bfloat16)
    s0 = None
    if init_std is not None:
        s0 = float(init_std) * torch.randn(len(lengths), H, HEAD_DIM, HEAD_DIM, generator=gen)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return PrefillCase(q, k, v, a, b, cu, s0, float("-inf"), SCALE, int(seed), name,
                       {"lengths": lengths})


# The five workloads: prefill configurations 0-3 and the decode sweep 4.
PREFILL_CONFIGS = {
    0: dict(name="prefill_T64_H2", num_heads=2, lower_bound=-5.0, init_std=None),
    1: dict(name="prefill_small_bh_T8192_H8", num_heads=8, lower_bound=-5.0, init_std=0.02),
    2: dict(name="prefill_varlen16_H32", num_heads=32, lower_bound=-5.0, init_std=0.02),
    3: dict(name="prefill_batch4x8192_H64_lb-8", num_heads=64, lower_bound=-8.0,
            init_std=None),
}


def _config_lengths(i: int, gen: torch.Generator):
    if i == 0:
        return [64]
    if i == 1:
        return [8192]
    if i == 2:
        while True:
            lens = torch.randint(256, 4097, (16,), generator=gen).tolist()
            if any(x % 32 for x in lens):
                return lens
    if i == 3:
        return [8192] * 4
    raise ValueError(f"no prefill configuration {i}")


def prefill_config(i: int, seed: Optional[int] = None) -> PrefillCase:
    """Prefill configuration i in 0..3 at full size (seed defaults to 20260 + i)."""
    seed = BASE_SEED + i if seed is None else int(seed)
    cfg = PREFILL_CONFIGS[i]
    lens = _config_lengths(i, torch.Generator().manual_seed(seed ^ 0x5EED))
    return make_prefill_case(lens, cfg["num_heads"], cfg["lower_bound"], cfg["init_std"],
                             seed, cfg["name"])


def make_decode_case(rows, num_heads=8, num_slots=4096, state_dtype=torch.float32,
                     init_std=0.02, seed=BASE_SEED + 4, name="", dk=HEAD_DIM,
                     dv=HEAD_DIM, with_pool=True) -> DecodeCase:
    """T=1 decode inputs: scattered unique slots into a random state pool.

    The bf16 pool holds the bf16 rounding of the same fp32 draw.  With
    ``with_pool=False`` the pool is not drawn (``pool`` is None) and every
    other tensor is unchanged.
    """
    gen = torch.Generator().manual_seed(int(seed))
    R, H = int(rows), int(num_heads)
    if R > num_slots:
        raise ValueError("rows exceed the pool size (slots must be unique)")
    q = _unit_rows(torch.randn(R, H, dk, generator=gen)).to(torch.bfloat16)
    k = _unit_rows(torch.randn(R, H, dk, generator=gen)).to(torch.bfloat16)
    v = torch.randn(R, H, dv, generator=gen).to(torch.bfloat16)
    g = (-torch.nn.functional.softplus(torch.randn(R, H, dk, generator=gen))).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn(R, H, generator=gen)).to(torch.bfloat16)
    slots = torch.randperm(int(num_slots), generator=gen)[:R].to(torch.int32)
    pool = None
    if with_pool:
        pool = make_decode_pool(num_slots, H, state_dtype, init_std, gen, dk, dv)
    return DecodeCase(q, k, v, g, beta, pool, slots, SCALE, int(seed), name)


def make_decode_raw_case(rows, num_heads=8, num_slots=4096, seed=BASE_SEED + 5,
                         qk_std=3.0) -> DecodeCase:
    """Decode inputs as a model hands them over before the input front-end:
    q, k ~ qk_std N(0, 1) (not normalised), v ~ N(0, 1), the gate tensor holds
    raw a ~ N(0, 1), beta holds logits ~ N(0, 1); all bf16.  Same draw order
    as make_decode_case; no pool is drawn."""
    gen = torch.Generator().manual_seed(int(seed))
    R, H = int(rows), int(num_heads)
    if R > num_slots:
        raise ValueError("rows exceed the pool size (slots must be unique)")
    q = (float(qk_std) * torch.randn(R, H, HEAD_DIM, generator=gen)).to(torch.bfloat16)
    k = (float(qk_std) * torch.randn(R, H, HEAD_DIM, generator=gen)).to(torch.bfloat16)
    v = torch.randn(R, H, HEAD_DIM, generator=gen).to(torch.bfloat16)
    a = torch.randn(R, H, HEAD_DIM, generator=gen).to(torch.bfloat16)
    b = torch.randn(R, H, generator=gen).to(torch.bfloat16)
    slots = torch.randperm(int(num_slots), generator=gen)[:R].to(torch.int32)
    return DecodeCase(q, k, v, a, b, None, slots, SCALE, int(seed), "raw")


def make_decode_pool(num_slots, num_heads, state_dtype=torch.float32, init_std=0.02,
                     gen=None, dk=HEAD_DIM, dv=HEAD_DIM) -> torch.Tensor:
    """State pool [num_slots, H, dk, dv]: init_std * N(0, 1) in fp32 (bf16: rounded)."""
    if gen is None or isinstance(gen, int):
        gen = torch.Generator().manual_seed(BASE_SEED + 4 if gen is None else int(gen))
    pool = float(init_std) * torch.randn(int(num_slots), int(num_heads), dk, dv, generator=gen)
    if state_dtype == torch.bfloat16:
        return pool.to(torch.bfloat16)
    if state_dtype != torch.float32:
        raise ValueError("state dtype must be float32 or bfloat16")
    return pool


def decode_config(rows: int, state_dtype=torch.float32, seed: Optional[int] = None,
                  num_slots: int = 4096) -> DecodeCase:
    """Decode configuration: H=8, 4096-slot pool, the given row count."""
    seed = BASE_SEED + 4 if seed is None else int(seed)
    tag = "f32" if state_dtype == torch.float32 else "bf16"
    return make_decode_case(rows, 8, num_slots, state_dtype, 0.02, seed,
                            f"decode_H8_rows{rows}_{tag}")
