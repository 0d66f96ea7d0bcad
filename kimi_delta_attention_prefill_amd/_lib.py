"""ctypes binding of ``libkda.so`` (include/kda.h).

Argument marshalling only: shapes, dtypes and devices are checked, output
buffers are allocated with PyTorch when the caller passes none, and the raw
device pointers plus the current HIP stream go to the C ABI.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import library_path

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE = -3
KDA_ERR_HIP = -4

ROUTE_AUTO = -1
ROUTE_SERIAL = 0
ROUTE_CHUNK = 1
ROUTE_SPLIT = 2
ROUTE_STREAM = 3

ANCHOR_FIXED = 0
ANCHOR_SPLIT16 = 1
ANCHOR_DATA = 2

STATE_F32 = 0
STATE_BF16 = 1

_lib = None


class KdaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class _Plan(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int32), ("anchor_mode", ctypes.c_int32),
                ("dv_split", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int64), ("anchor_log2", ctypes.c_float),
                ("windows", ctypes.c_int32), ("window_chunks", ctypes.c_int32)]


class _FrontEnd(ctypes.Structure):
    _fields_ = [("gate_mode", ctypes.c_int32), ("lower_bound", ctypes.c_float),
                ("beta_logits", ctypes.c_int32), ("normalize_qk", ctypes.c_int32),
                ("norm_eps", ctypes.c_float)]


GATE_LOG, GATE_LOWER_BOUND, GATE_SOFTPLUS = 0, 1, 2


@dataclass
class FrontEnd:
    """Input front-end of kda_decode_ex / kda_prefill_ex (include/kda.h:
    kda_frontend): gate_mode GATE_LOG (g is the log-decay), GATE_LOWER_BOUND
    (g holds a; decay lower_bound * sigmoid(a)) or GATE_SOFTPLUS (decay
    -softplus(a)); beta_logits: beta = sigmoid(beta); normalize_qk: q, k scaled
    by 1 / sqrt(sum x^2 + norm_eps)."""
    gate_mode: int = GATE_LOG
    lower_bound: float = 0.0
    beta_logits: bool = False
    normalize_qk: bool = False
    norm_eps: float = 0.0

    def _c(self):
        return _FrontEnd(int(self.gate_mode), float(self.lower_bound), int(bool(self.beta_logits)),
                         int(bool(self.normalize_qk)), float(self.norm_eps))


def _fe_ptr(fe):
    return None if fe is None else ctypes.byref(fe._c())


@dataclass
class Plan:
    route: int
    anchor_mode: int
    dv_split: int
    block_threads: int
    grid_blocks: int
    anchor_log2: float
    windows: int = 1
    window_chunks: int = 0


def load():
    """Load libkda.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m kimi_delta_attention_prefill_amd.build`"
                          " (or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.kda_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, f32, vp, vp,
                                vp, vp, sz, vp]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, f32,
                                   ctypes.POINTER(_FrontEnd), vp, vp, vp, vp, sz, vp]
    lib.kda_prefill_ex.restype = ctypes.c_int
    lib.kda_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, f32,
                                        vp, vp, vp, vp]
    lib.kda_prefill_noalloc.restype = ctypes.c_int
    lib.kda_prefill_workspace_size.argtypes = [i32, i64, i32]
    lib.kda_prefill_workspace_size.restype = sz
    lib.kda_prefill_plan.argtypes = [i32, i64, i32, f32, i32, i32, ctypes.POINTER(_Plan)]
    lib.kda_prefill_plan.restype = ctypes.c_int
    lib.kda_set_prefill_route.argtypes = [i32]
    lib.kda_set_prefill_route.restype = ctypes.c_int
    lib.kda_prefill_prepare.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, vp,
                                        sz, vp]
    lib.kda_prefill_prepare.restype = ctypes.c_int
    lib.kda_prefill_chain.argtypes = [vp, i32, i64, i32, f32, vp, vp, vp, vp, sz, vp]
    lib.kda_prefill_chain.restype = ctypes.c_int
    lib.kda_prefill_records_size.argtypes = [i32, i64, i32]
    lib.kda_prefill_records_size.restype = sz
    lib.kda_prefill_pool.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, f32, vp,
                                     i64, vp, vp, i32, vp, vp, sz, vp]
    lib.kda_prefill_pool.restype = ctypes.c_int
    lib.kda_prefill_pool_ex.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, f32,
                                        ctypes.POINTER(_FrontEnd), vp, i32, i64, i64, vp, vp, i32,
                                        vp, vp, sz, vp]
    lib.kda_prefill_pool_ex.restype = ctypes.c_int
    lib.kda_prefill_checkpoint_slots.argtypes = [i32, i64, i32]
    lib.kda_prefill_checkpoint_slots.restype = sz
    lib.kda_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, vp, i32, i32, i32, i32, f32, vp, vp]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode_ex.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, vp, i32, i32, i32, i32,
                                  f32, ctypes.POINTER(_FrontEnd), vp, vp]
    lib.kda_decode_ex.restype = ctypes.c_int
    lib.kda_check_prefill_inputs.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, f32, vp, vp]
    lib.kda_check_prefill_inputs.restype = ctypes.c_int
    lib.kda_check_slots.argtypes = [vp, i32, i64, vp, vp]
    lib.kda_check_slots.restype = ctypes.c_int
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load().kda_last_error().decode()


def _check(rc: int):
    if rc != KDA_OK:
        raise KdaError(rc, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _pool_layout(pool, H, D, device):
    """(state dtype code, slot stride) of a [num_slots, H, D, D] state pool.

    Each slot's [H, D, D] block must be dense; the slots themselves may sit
    at a larger stride (the padded layout, e.g. one layer's view of a pool
    [num_slots, layers, H, D, D]).  Stride 0 means dense."""
    if pool.dtype == torch.float32:
        sd = STATE_F32
    elif pool.dtype == torch.bfloat16:
        sd = STATE_BF16
    else:
        raise TypeError("state_pool must be float32 or bfloat16")
    if tuple(pool.shape[1:]) != (H, D, D) or pool.dim() != 4:
        raise ValueError(f"state_pool: expected shape (num_slots, {H}, {D}, {D}), "
                         f"got {tuple(pool.shape)}")
    if pool.device != device:
        raise ValueError(f"state_pool: expected device {device}, got {pool.device}")
    dense = H * D * D
    if pool.stride()[1:] != (D * D, D, 1) or (pool.shape[0] > 1 and pool.stride(0) < dense):
        raise ValueError("state_pool: each slot's [H, D, D] block must be dense and slots "
                         "must not overlap")
    stride = pool.stride(0) if pool.shape[0] > 1 else dense
    return sd, (0 if stride == dense else stride)


def workspace_size(num_seqs: int, total_tokens: int, num_heads: int) -> int:
    return int(load().kda_prefill_workspace_size(num_seqs, total_tokens, num_heads))


def plan(num_seqs: int, total_tokens: int, num_heads: int, lower_bound: float,
         num_cus: int = 0, route: int = ROUTE_AUTO) -> Plan:
    """What kda_prefill would launch (pure host function)."""
    p = _Plan()
    _check(load().kda_prefill_plan(num_seqs, total_tokens, num_heads, lower_bound, num_cus, route,
                                   ctypes.byref(p)))
    return Plan(p.route, p.anchor_mode, p.dv_split, p.block_threads, p.grid_blocks, p.anchor_log2,
                p.windows, p.window_chunks)


def set_prefill_route(route: int) -> None:
    """Force a prefill route process-wide (ROUTE_AUTO restores automatic selection)."""
    _check(load().kda_set_prefill_route(route))


def prefill(q, k, v, g, beta, cu_seqlens, *, scale, lower_bound, initial_state=None,
            final_state=None, out=None, workspace=None, stream=None, frontend=None):
    """Packed varlen KDA prefill on the GPU.

    ``lower_bound``: the gate bound (< 0), or ``float("-inf")`` for an
    unbounded gate.  ``frontend``: a :class:`FrontEnd` (kda_prefill_ex) or
    None (kda_prefill).

    ``workspace``: a device uint8 tensor of at least ``workspace_size(N, T, H)``
    bytes (allocated here when None and the chosen route needs one).

    q, k, v, g: bf16 [T, H, 128]; beta: bf16 [T, H]; cu_seqlens: int32 [N+1]
    (device); initial_state: fp32 [N, H, 128, 128] or None (zeros).
    ``final_state``: an fp32 [N, H, 128, 128] tensor to write into, True to
    allocate one, or None/False to skip it.  Returns (out, final_state).
    """
    dev = q.device
    T, H, D = q.shape
    N = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _need(t, name, torch.bfloat16, (T, H, D), dev)
    _need(beta, "beta", torch.bfloat16, (T, H), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, D, D), dev)
    if final_state is True:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, D, D), dev)
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H, D), dev)
    if workspace is None:
        need = workspace_size(N, T, H)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if frontend is None:
        _check(load().kda_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                  N, T, H, D, D, float(scale), float(lower_bound),
                                  _ptr(initial_state), _ptr(final_state), _ptr(out), _ptr(workspace),
                                  ws_bytes, _stream(stream)))
    else:
        _check(load().kda_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(cu_seqlens), N, T, H, D, D, float(scale),
                                     float(lower_bound), _fe_ptr(frontend), _ptr(initial_state),
                                     _ptr(final_state), _ptr(out), _ptr(workspace), ws_bytes,
                                     _stream(stream)))
    return out, final_state


def prefill_noalloc(q, k, v, g, beta, cu_seqlens, *, scale, lower_bound, initial_state=None,
                    final_state=None, out=None, stream=None):
    """kda_prefill_noalloc: :func:`prefill` without a workspace; the split
    route's workspace is the library's static device scratch (raises
    KdaError with KDA_ERR_WORKSPACE when the problem needs more).  Outputs
    and the final state as in :func:`prefill` (allocated here when not
    given).  Returns (out, final_state)."""
    dev = q.device
    T, H, D = q.shape
    N = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _need(t, name, torch.bfloat16, (T, H, D), dev)
    _need(beta, "beta", torch.bfloat16, (T, H), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, D, D), dev)
    if final_state is True:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, D, D), dev)
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H, D), dev)
    _check(load().kda_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(cu_seqlens), N, T, H, D, D, float(scale),
                                      float(lower_bound), _ptr(initial_state), _ptr(final_state),
                                      _ptr(out), _stream(stream)))
    return out, final_state


NOALLOC_SCRATCH_BYTES = 128 << 20   # KDA_NOALLOC_SCRATCH_BYTES


def checkpoint_slots(num_seqs: int, total_tokens: int, checkpoint_tokens: int) -> int:
    """Slots ([H, 128, 128] each) a checkpoint buffer of prefill_pool must hold."""
    return int(load().kda_prefill_checkpoint_slots(num_seqs, total_tokens, checkpoint_tokens))


def prefill_pool(q, k, v, g, beta, cu_seqlens, slot_indices, state_pool, *, scale, lower_bound,
                 checkpoints=None, checkpoint_tokens=64, out=None, workspace=None, stream=None,
                 frontend=None):
    """Packed varlen prefill whose states live in ``state_pool`` (fp32 or
    bf16 [num_slots, H, 128, 128], updated in place; each slot dense, the
    slots dense or at a larger stride (a view); None: zero start, nothing
    stored), one ``slot_indices`` entry (int32, device) per sequence.

    ``checkpoints``: an fp32 [checkpoint_slots(N, T, checkpoint_tokens), H, 128, 128]
    tensor to fill, True to allocate one (zero-filled), or None for none.
    Returns (out, checkpoints).
    """
    dev = q.device
    T, H, D = q.shape
    N = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _need(t, name, torch.bfloat16, (T, H, D), dev)
    _need(beta, "beta", torch.bfloat16, (T, H), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    _need(slot_indices, "slot_indices", torch.int32, (N,), dev)
    num_slots, sd, stride = 0, STATE_F32, 0
    if state_pool is not None:
        sd, stride = _pool_layout(state_pool, H, D, dev)
        num_slots = state_pool.shape[0]
    if checkpoints is True:
        checkpoints = torch.zeros((checkpoint_slots(N, T, checkpoint_tokens), H, D, D),
                                  dtype=torch.float32, device=dev)
    if checkpoints is not None:
        _need(checkpoints, "checkpoints", torch.float32,
              (checkpoint_slots(N, T, checkpoint_tokens), H, D, D), dev)
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H, D), dev)
    if workspace is None:
        need = workspace_size(N, T, H)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kda_prefill_pool_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(cu_seqlens), N, T, H, D, D, float(scale),
                                      float(lower_bound), _fe_ptr(frontend), _ptr(state_pool), sd,
                                      num_slots, stride, _ptr(slot_indices), _ptr(checkpoints),
                                      int(checkpoint_tokens) if checkpoints is not None else 0,
                                      _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, checkpoints


def records_size(num_seqs: int, total_tokens: int, num_heads: int) -> int:
    """Bytes of chunk records kda_prefill_prepare / kda_prefill_chain need."""
    return int(load().kda_prefill_records_size(num_seqs, total_tokens, num_heads))


def prefill_prepare(q, k, v, g, beta, cu_seqlens, *, lower_bound, records=None, stream=None):
    """First pass of the two-pass prefill: chunk records into ``records``
    (a device uint8 tensor of at least ``records_size(N, T, H)`` bytes,
    allocated here when None).  Returns ``records``."""
    dev = q.device
    T, H, D = q.shape
    N = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _need(t, name, torch.bfloat16, (T, H, D), dev)
    _need(beta, "beta", torch.bfloat16, (T, H), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if records is None:
        records = torch.empty(max(records_size(N, T, H), 16), dtype=torch.uint8, device=dev)
    _check(load().kda_prefill_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(cu_seqlens), N, T, H, D, D, float(lower_bound),
                                      _ptr(records), records.numel() * records.element_size(),
                                      _stream(stream)))
    return records


def prefill_chain(records, cu_seqlens, num_heads, *, scale, total_tokens, initial_state=None,
                  final_state=None, out=None, stream=None):
    """Second pass of the two-pass prefill: the serial chain over ``records``.
    ``final_state`` as in :func:`prefill`.  Returns (out, final_state)."""
    dev = records.device
    N = cu_seqlens.numel() - 1
    T, H, D = int(total_tokens), int(num_heads), 128
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, D, D), dev)
    if final_state is True:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, D, D), dev)
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H, D), dev)
    _check(load().kda_prefill_chain(_ptr(cu_seqlens), N, T, H, float(scale), _ptr(initial_state),
                                    _ptr(final_state), _ptr(out), _ptr(records),
                                    records.numel() * records.element_size(), _stream(stream)))
    return out, final_state


def decode(q, k, v, g, beta, state_pool, slot_indices, *, scale, out=None, stream=None,
           frontend=None):
    """One T=1 step per row against ``state_pool`` (fp32 or bf16), in place.

    q, k, v, g: bf16 [rows, H, 128]; beta: bf16 [rows, H];
    state_pool: [num_slots, H, 128, 128], each slot dense, slots dense or at a
    larger stride (a view); slot_indices: int32 [rows].
    ``frontend``: a :class:`FrontEnd` (kda_decode_ex) or None (kda_decode).
    Returns out (bf16 [rows, H, 128]).
    """
    dev = q.device
    R, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _need(t, name, torch.bfloat16, (R, H, D), dev)
    _need(beta, "beta", torch.bfloat16, (R, H), dev)
    _need(slot_indices, "slot_indices", torch.int32, (R,), dev)
    sd, stride = _pool_layout(state_pool, H, D, dev)
    if out is None:
        out = torch.empty((R, H, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (R, H, D), dev)
    if frontend is None and stride == 0:
        _check(load().kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                 sd, state_pool.shape[0], _ptr(slot_indices), R, H, D, D,
                                 float(scale), _ptr(out), _stream(stream)))
    else:
        _check(load().kda_decode_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state_pool), sd, state_pool.shape[0], stride,
                                    _ptr(slot_indices), R, H, D, D, float(scale),
                                    _fe_ptr(frontend), _ptr(out),
                                    _stream(stream)))
    return out


CHECK_NAMES = ("cu_seqlens", "gate_range", "beta_range", "qkv_finite", "slots_unique",
               "gate_steep")


def check_prefill_inputs(q, k, v, g, beta, cu_seqlens, *, lower_bound, stream=None):
    """Device check of kda_prefill's documented preconditions (debugging and
    tests; synchronises).  Returns {check name: True when it fails}."""
    dev = q.device
    T, H, _ = q.shape
    N = cu_seqlens.numel() - 1
    flags = torch.full((6,), -1, dtype=torch.int32, device=dev)
    _check(load().kda_check_prefill_inputs(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                           _ptr(cu_seqlens), N, T, H, float(lower_bound),
                                           _ptr(flags), _stream(stream)))
    torch.cuda.synchronize(dev)
    f = flags.cpu().tolist()
    return {CHECK_NAMES[i]: bool(f[i]) for i in (0, 1, 2, 3, 5)}


def check_slots(slot_indices, num_slots, *, stream=None):
    """Device check that the slot indices in [0, num_slots) are distinct
    (debugging and tests; synchronises).  Returns True when they are not."""
    flags = torch.full((6,), -1, dtype=torch.int32, device=slot_indices.device)
    _check(load().kda_check_slots(_ptr(slot_indices), slot_indices.numel(), int(num_slots),
                                  _ptr(flags), _stream(stream)))
    torch.cuda.synchronize(slot_indices.device)
    return bool(flags[4].item())

