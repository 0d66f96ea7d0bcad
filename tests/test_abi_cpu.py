"""CPU-only checks of the C ABI: the library loads, exports what include/kda.h
declares, plans routes as a pure function, and rejects bad arguments on the
host before anything is enqueued (no compute call needs a GPU here)."""
import ctypes
import os
import re

import pytest

import kimi_delta_attention_prefill_amd as kda
from kimi_delta_attention_prefill_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = kda.load()
    names = _declared_functions()
    assert {"kda_prefill", "kda_decode", "kda_last_error"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"libkda.so does not export {name}"


def test_abi_version_matches_header():
    text = open(HEADER).read()
    ver = int(re.search(r"#define KDA_ABI_VERSION (\d+)", text).group(1))
    assert kda.load().kda_abi_version() == ver


def test_plan_anchor_mode_boundary():
    # fixed anchor iff 16 |lb| log2(e) <= 116 (the budget that keeps the bf16
    # low halves of the anchored operands)  <=>  |lb| <= 5.0254...
    assert kda.plan(1, 64, 2, -5.0, 256).anchor_mode == kda.ANCHOR_FIXED
    assert kda.plan(1, 64, 2, -5.02, 256).anchor_mode == kda.ANCHOR_FIXED
    assert kda.plan(1, 64, 2, -5.03, 256).anchor_mode == kda.ANCHOR_SPLIT16
    assert kda.plan(4, 32768, 64, -8.0, 256).anchor_mode == kda.ANCHOR_SPLIT16
    # 16-token anchors at the integer h' nearest h = 8 lb log2(e): factors up to
    # 2^|h'| and 2^|2h - h'|, both <= 116 down to |lb| ~ 10.05
    assert kda.plan(1, 64, 2, -10.0, 256).anchor_mode == kda.ANCHOR_SPLIT16
    assert kda.plan(1, 64, 2, -10.05, 256).anchor_mode == kda.ANCHOR_SPLIT16
    assert kda.plan(1, 64, 2, -10.1, 256).anchor_mode == kda.ANCHOR_DATA
    assert kda.plan(1, 64, 2, -10.875, 256).anchor_mode == kda.ANCHOR_DATA
    p = kda.plan(1, 64, 2, -5.0, 256)
    assert abs(p.anchor_log2 - 16 * -5.0 * 1.4426950408889634) < 1e-4


@pytest.mark.parametrize("route", [kda.ROUTE_SERIAL, kda.ROUTE_CHUNK, kda.ROUTE_SPLIT, kda.ROUTE_STREAM])
def test_plan_grid_covers_every_unit(route):
    for N, H, cus in ((1, 8, 256), (16, 32, 256), (4, 64, 256), (1, 1, 256), (3, 5, 80)):
        p = kda.plan(N, 100 * N, H, -5.0, cus, route)
        assert p.route == route
        assert p.dv_split >= 1 and 128 % p.dv_split == 0
        assert p.grid_blocks == N * H * p.dv_split
        assert p.block_threads % 64 == 0 and 64 <= p.block_threads <= 1024


def test_plan_rejects_bad_inputs():
    for args in ((-1, 0, 1, -5.0), (1, -1, 1, -5.0), (1, 0, 0, -5.0), (1, 0, 1, 0.0),
                 (1, 0, 1, float("nan")), (1, 0, 1, float("inf")), (1, 0, 1, 1.0)):
        with pytest.raises(kda.KdaError) as e:
            kda.plan(*args, num_cus=256)
        assert e.value.code == _lib.KDA_ERR_INVALID_ARGUMENT
        assert kda.last_error()
    with pytest.raises(kda.KdaError):
        kda.plan(1, 0, 1, -5.0, 256, route=7)


def test_plan_unbounded_gate_uses_data_anchors():
    # lower_bound = -inf: no bound, each 16-token half anchored at its own range
    for route in (kda.ROUTE_CHUNK, kda.ROUTE_SPLIT):
        p = kda.plan(2, 3000, 4, float("-inf"), 256, route)
        assert p.anchor_mode == kda.ANCHOR_DATA and p.anchor_log2 == 0.0
    # the fused route runs data anchors on 64-column blocks only
    assert kda.plan(16, 35000, 32, float("-inf"), 256, kda.ROUTE_CHUNK).dv_split == 2
    assert kda.plan(16, 35000, 32, -5.0, 256, kda.ROUTE_CHUNK).dv_split == 1
    assert kda.plan(1, 64, 2, -5.0, 256).anchor_mode == kda.ANCHOR_FIXED


def test_set_route_validates():
    with pytest.raises(kda.KdaError):
        kda.set_prefill_route(5)
    kda.set_prefill_route(kda.ROUTE_AUTO)


def _prefill_raw(**over):
    a = dict(q=16, k=16, v=16, g=16, beta=16, cu=16, N=1, T=4, H=1, dk=128, dv=128, scale=1.0,
             lb=-5.0, s0=None, s1=None, out=16, ws=None, ws_bytes=0)
    a.update(over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return kda.load().kda_prefill(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
                                  P(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"], a["scale"],
                                  a["lb"], P(a["s0"]), P(a["s1"]), P(a["out"]), P(a["ws"]),
                                  a["ws_bytes"], None)


def test_prefill_host_validation():
    E, U = _lib.KDA_ERR_INVALID_ARGUMENT, _lib.KDA_ERR_UNSUPPORTED
    # Every case below is rejected before any device work (pointers are never dereferenced).
    assert _prefill_raw(dk=64) == U
    assert _prefill_raw(dv=256) == U
    assert _prefill_raw(H=0) == E
    assert _prefill_raw(N=-1) == E
    assert _prefill_raw(T=-1) == E
    assert _prefill_raw(T=2 ** 31) == E
    assert _prefill_raw(lb=0.0) == E
    assert _prefill_raw(lb=float("nan")) == E
    assert _prefill_raw(scale=float("inf")) == E
    assert _prefill_raw(cu=None) == E
    assert _prefill_raw(q=None) == E
    assert _prefill_raw(out=None) == E
    assert _prefill_raw(q=0x1008) == E          # misaligned bf16 tensor
    assert _prefill_raw(beta=0x1001) == E       # misaligned beta
    assert _prefill_raw(s0=0x1004) == E         # misaligned state
    assert _prefill_raw(s0=0x10000, s1=0x10000 + 4096) == E   # partial overlap
    assert "overlap" in kda.last_error()
    # N == 0 is a valid no-op that touches nothing.
    assert _prefill_raw(N=0, q=None, k=None, v=None, g=None, beta=None, cu=None, out=None) == 0


def _decode_raw(**over):
    a = dict(q=16, k=16, v=16, g=16, beta=16, pool=16, dtype=0, slots_n=4, idx=16, rows=2, H=8,
             dk=128, dv=128, scale=1.0, out=16)
    a.update(over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return kda.load().kda_decode(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
                                 P(a["pool"]), a["dtype"], a["slots_n"], P(a["idx"]), a["rows"],
                                 a["H"], a["dk"], a["dv"], a["scale"], P(a["out"]), None)


def test_decode_host_validation():
    E, U = _lib.KDA_ERR_INVALID_ARGUMENT, _lib.KDA_ERR_UNSUPPORTED
    assert _decode_raw(dk=64) == U
    assert _decode_raw(dtype=3) == E
    assert _decode_raw(rows=-1) == E
    assert _decode_raw(H=0) == E
    assert _decode_raw(slots_n=0) == E
    assert _decode_raw(scale=float("nan")) == E
    assert _decode_raw(pool=None) == E
    assert _decode_raw(idx=None) == E
    assert _decode_raw(pool=0x1008) == E
    assert _decode_raw(idx=0x1002) == E
    assert _decode_raw(rows=0, q=None, pool=None, idx=None, out=None) == 0


def test_check_entry_points_host_validation():
    """kda_check_prefill_inputs / kda_check_slots reject bad arguments on the
    host, before anything is enqueued (the fake pointers are never touched)."""
    lib = kda.load()
    E = _lib.KDA_ERR_INVALID_ARGUMENT
    P = ctypes.c_void_p
    A = P(0x1000)

    def pre(N=1, T=64, H=2, lb=-5.0, flags=A, cu=A, q=A):
        return lib.kda_check_prefill_inputs(q, A, A, A, A, cu, N, T, H, lb, flags, None)

    assert pre(N=-1) == E
    assert pre(T=-1) == E
    assert pre(H=0) == E
    assert pre(lb=0.0) == E
    assert pre(lb=float("nan")) == E
    assert pre(flags=None) == E
    assert pre(flags=P(0x1002)) == E
    assert pre(cu=None) == E
    assert pre(q=None) == E
    assert pre(q=P(0x1001)) == E
    assert "kda_check_prefill_inputs" in kda.last_error()

    def slots(rows=4, n=16, idx=A, flags=A):
        return lib.kda_check_slots(idx, rows, n, flags, None)

    assert slots(rows=-1) == E
    assert slots(n=0) == E
    assert slots(flags=None) == E
    assert slots(idx=None) == E
    assert slots(idx=P(0x1002)) == E


def test_decode_frontend_host_validation():
    lib = kda.load()
    E = _lib.KDA_ERR_INVALID_ARGUMENT
    P = ctypes.c_void_p

    def call(fe, stride=0, dtype=0):
        ref = None if fe is None else ctypes.byref(fe._c())
        return lib.kda_decode_ex(P(16), P(16), P(16), P(16), P(16), P(16), dtype, 4, stride, P(16),
                                 0, 8, 128, 128, 1.0, ref, P(16), None)

    assert call(None) == 0                                       # rows = 0: a no-op
    assert call(kda.FrontEnd()) == 0
    assert call(kda.FrontEnd(gate_mode=kda.GATE_SOFTPLUS, beta_logits=True, normalize_qk=True,
                             norm_eps=1e-6)) == 0
    assert call(kda.FrontEnd(gate_mode=3)) == E
    assert "gate mode" in kda.last_error()
    assert call(kda.FrontEnd(gate_mode=kda.GATE_LOWER_BOUND, lower_bound=0.0)) == E
    assert call(kda.FrontEnd(gate_mode=kda.GATE_LOWER_BOUND, lower_bound=float("-inf"))) == E
    assert call(kda.FrontEnd(gate_mode=kda.GATE_LOWER_BOUND, lower_bound=-5.0)) == 0
    assert call(kda.FrontEnd(normalize_qk=True, norm_eps=-1e-6)) == E
    assert call(kda.FrontEnd(normalize_qk=True, norm_eps=float("nan"))) == E
    # slot stride: 0 (dense) or >= H * 128 * 128 elements and a multiple of 16 bytes
    dense = 8 * 128 * 128
    assert call(None, stride=dense) == 0 and call(None, stride=3 * dense) == 0
    assert call(None, stride=dense + 4) == 0                     # fp32: 16 bytes
    assert call(None, stride=dense + 4, dtype=1) == E            # bf16: 8 bytes
    assert "slot_stride" in kda.last_error()
    assert call(None, stride=dense + 8, dtype=1) == 0
    assert call(None, stride=dense - 4) == E                     # overlapping slots
    assert call(None, stride=-dense) == E


def test_auto_route_and_workspace():
    # few (sequence, head) units: two-pass split route; many: fused chunk route
    assert kda.plan(1, 8192, 8, -5.0, 256).route == kda.ROUTE_SPLIT
    # many short sequences (multi-token decode): the stream route, up to 4
    # tokens per sequence on average, up to 8 with at least one unit per CU
    assert kda.plan(4096, 4 * 4096, 8, float("-inf"), 256).route == kda.ROUTE_STREAM
    assert kda.plan(64, 2 * 64, 8, -5.0, 256).route == kda.ROUTE_STREAM
    assert kda.plan(1, 4, 8, -5.0, 256).route == kda.ROUTE_STREAM
    assert kda.plan(4096, 8 * 4096, 8, float("-inf"), 256).route == kda.ROUTE_STREAM
    assert kda.plan(1, 8, 8, -5.0, 256).route == kda.ROUTE_CHUNK          # 8 units only
    assert kda.plan(4096, 9 * 4096, 8, float("-inf"), 256).route == kda.ROUTE_CHUNK
    assert kda.plan(1, 5, 2, -5.0, 256).route == kda.ROUTE_CHUNK
    # at most three chunks in the batch: the fused route's serial loop is shorter
    assert kda.plan(1, 64, 2, -5.0, 256).route == kda.ROUTE_CHUNK
    assert kda.plan(3, 96, 8, -5.0, 256).route == kda.ROUTE_CHUNK
    assert kda.plan(1, 97, 2, -5.0, 256).route == kda.ROUTE_SPLIT
    assert kda.plan(16, 35000, 32, -5.0, 256).route == kda.ROUTE_CHUNK
    assert kda.plan(4, 32768, 64, -8.0, 256).route == kda.ROUTE_CHUNK
    # crossover against the fused pipeline: up to a quarter of the CUs in units
    assert kda.plan(1, 8192, 64, -5.0, 256).route == kda.ROUTE_SPLIT
    assert kda.plan(1, 8192, 65, -5.0, 256).route == kda.ROUTE_CHUNK
    assert kda.plan(4, 16384, 24, -5.0, 256).route == kda.ROUTE_CHUNK     # 96 units
    assert kda.plan(1, 8192, 97, -5.0, 256).route == kda.ROUTE_CHUNK
    assert kda.plan(2, 16384, 64, -5.0, 256).route == kda.ROUTE_CHUNK
    try:
        kda.set_prefill_route(kda.ROUTE_SPLIT)
        # one long sequence: records plus the window states (E and P per window and head)
        assert kda.workspace_size(1, 8192, 8) == ((1 + 8192 // 32 + 1) * 8 * 49152
                                                  + 1 * 8 * 5 * 2 * 65536)
        assert kda.workspace_size(3, 100, 2) == (3 + 3 + 1) * 2 * 49152
        kda.set_prefill_route(kda.ROUTE_CHUNK)
        assert kda.workspace_size(16, 40000, 32) == 0
        kda.set_prefill_route(kda.ROUTE_SERIAL)
        assert kda.workspace_size(1, 8192, 8) == 0
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)


def test_split_route_requires_workspace():
    try:
        kda.set_prefill_route(kda.ROUTE_SPLIT)
        rc = _prefill_raw(ws=None, ws_bytes=0)
        assert rc == _lib.KDA_ERR_WORKSPACE and "workspace" in kda.last_error()
        rc = _prefill_raw(ws=0x10000, ws_bytes=100)
        assert rc == _lib.KDA_ERR_WORKSPACE
    finally:
        kda.set_prefill_route(kda.ROUTE_AUTO)


def test_two_pass_host_validation():
    lib = kda.load()
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    need = kda.records_size(1, 4, 1)
    assert need == (1 + 0 + 1) * 1 * 49152
    assert kda.records_size(3, 100, 2) == (3 + 3 + 1) * 2 * 49152
    assert kda.records_size(0, 0, 1) == 0 and kda.records_size(1, -1, 1) == 0

    def prep(**o):
        a = dict(q=16, k=16, v=16, g=16, beta=16, cu=16, N=1, T=4, H=1, dk=128, dv=128, lb=-5.0,
                 rec=0x10000, nbytes=need)
        a.update(o)
        return lib.kda_prefill_prepare(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
                                       P(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"], a["lb"],
                                       P(a["rec"]), a["nbytes"], None)

    def chain(**o):
        a = dict(cu=16, N=1, T=4, H=1, scale=1.0, s0=None, s1=None, out=16, rec=0x10000,
                 nbytes=need)
        a.update(o)
        return lib.kda_prefill_chain(P(a["cu"]), a["N"], a["T"], a["H"], a["scale"], P(a["s0"]),
                                     P(a["s1"]), P(a["out"]), P(a["rec"]), a["nbytes"], None)

    E, U, W = _lib.KDA_ERR_INVALID_ARGUMENT, _lib.KDA_ERR_UNSUPPORTED, _lib.KDA_ERR_WORKSPACE
    assert prep(dk=64) == U
    assert prep(lb=0.0) == E
    assert prep(q=None) == E and prep(q=0x1008) == E and prep(cu=None) == E
    assert prep(rec=None) == W and "workspace" in kda.last_error()
    assert prep(nbytes=need - 1) == W
    assert prep(rec=0x10008) == E
    assert prep(N=0, q=None, cu=None, rec=None, nbytes=0) == 0
    assert chain(scale=float("nan")) == E
    assert chain(out=None) == E and chain(cu=None) == E
    assert chain(s0=0x20000, s1=0x20000 + 4096) == E and "overlap" in kda.last_error()
    assert chain(rec=None) == W and chain(nbytes=100) == W
    assert chain(N=0, cu=None, out=None, rec=None, nbytes=0) == 0


def test_plan_windows():
    # one sequence whose chain would use few CUs is cut into windows such that
    # phase A (1 + 2 (W - 2) chains) and phase C (W - 1 chains) fit two blocks per CU
    p = kda.plan(1, 8192, 8, -5.0, 256, kda.ROUTE_SPLIT)
    assert (p.windows, p.window_chunks) == (5, 52)
    assert 64 * (1 + 2 * (p.windows - 2)) <= 512 and 64 * (p.windows - 1) <= 512
    p = kda.plan(1, 3000, 3, -8.0, 256, kda.ROUTE_SPLIT)
    assert p.windows == 8 and p.window_chunks == 12          # 94 chunks: 7 x 12 + 10
    assert (p.windows - 1) * p.window_chunks < 94 <= p.windows * p.window_chunks
    p = kda.plan(1, 1000, 8, -5.0, 256, kda.ROUTE_SPLIT)   # 32 chunks: windows of >= 8 chunks
    assert (p.windows, p.window_chunks) == (4, 8)
    for args in ((1, 64, 2), (2, 345, 4), (1, 8192, 32), (1, 700, 8), (8, 4000, 4),
                 (4, 4 * 4096, 4)):
        p = kda.plan(*args, -5.0, 256, kda.ROUTE_SPLIT)
        assert (p.windows, p.window_chunks) == (1, 0), args   # too short or too many units
    # (4 x 4096 at H = 4 would get three windows of 43 chunks: not worth the carry)
    assert kda.plan(1, 8192, 8, -5.0, 256, kda.ROUTE_CHUNK).windows == 1
    # several sequences: W from the (sequence, head) count and the average
    # length; each sequence is cut by its own length on the device, into
    # max(8, ceil(chunks / W)) chunks per window (reported for a sequence as
    # long as the batch)
    p = kda.plan(2, 2 * 8192, 8, -5.0, 256, kda.ROUTE_SPLIT)      # 16 units, 128 chain tiles
    assert (p.windows, p.window_chunks) == (3, 171)
    assert 128 * (1 + 2 * (p.windows - 2)) <= 512 and 128 * (p.windows - 1) <= 512
    p = kda.plan(2, 3000 + 13384, 8, -5.0, 256, kda.ROUTE_SPLIT)
    assert p.windows == 3
    p = kda.plan(3, 2000 + 4100 + 777, 2, -8.0, 256, kda.ROUTE_SPLIT)
    assert p.windows == 6                                          # 6 units: 48 chain tiles
    assert kda.workspace_size(3, 6877, 2) == (
        (3 + 6877 // 32 + 1) * 2 * 49152 + 3 * 2 * p.windows * 2 * 65536)


def test_pool_prefill_host_validation():
    lib = kda.load()
    P = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(**o):
        a = dict(q=16, k=16, v=16, g=16, beta=16, cu=16, N=2, T=4, H=1, dk=128, dv=128, scale=1.0,
                 lb=-5.0, pool=0x10000, slots_n=4, idx=16, ck=None, ckt=0, out=16, ws=None,
                 ws_bytes=0)
        a.update(o)
        return lib.kda_prefill_pool(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
                                    P(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                    a["scale"], a["lb"], P(a["pool"]), a["slots_n"], P(a["idx"]),
                                    P(a["ck"]), a["ckt"], P(a["out"]), P(a["ws"]), a["ws_bytes"],
                                    None)

    E, U = _lib.KDA_ERR_INVALID_ARGUMENT, _lib.KDA_ERR_UNSUPPORTED
    assert call(dk=64) == U
    assert call(slots_n=0) == E
    assert call(pool=0x10008) == E
    assert call(idx=None) == E and call(idx=0x1002) == E
    assert call(ck=0x20000, ckt=48) == E and "multiple of 32" in kda.last_error()
    assert call(ck=0x20000, ckt=0) == E
    assert call(ck=0x20008, ckt=64) == E
    assert call(out=None) == E
    assert call(N=0, q=None, cu=None, idx=None, out=None) == 0

    def call_ex(stride, dtype=0, N=0):
        return lib.kda_prefill_pool_ex(P(16), P(16), P(16), P(16), P(16), P(16), N, 4, 1, 128,
                                       128, 1.0, -5.0, None, P(0x10000), dtype, 4, stride,
                                       P(16), None, 0, P(16), None, 0, None)

    dense = 128 * 128
    assert call_ex(0) == 0 and call_ex(dense) == 0 and call_ex(2 * dense + 4) == 0
    assert call_ex(dense + 4, dtype=1) == E and "slot_stride" in kda.last_error()
    assert call_ex(dense - 8) == E and call_ex(-1) == E
    assert call_ex(0, dtype=2) == E
    assert kda.checkpoint_slots(3, 1000, 64) == 3 + 1000 // 64 + 1
    assert kda.checkpoint_slots(1, 8192, 64) == 1 + 128 + 1
    assert kda.checkpoint_slots(1, 10, 0) == 0


def test_header_is_plain_c_and_links(tmp_path):
    """include/kda.h compiles as C11 and a C program links against libkda.so and
    calls it (host-only entry points: no device is touched)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_kda.c"
    src.write_text(r'''
#include <stdio.h>
#include "kda.h"
int main(void) {
  kda_frontend fe = {KDA_GATE_SOFTPLUS, 0.0f, 1, 1, 1e-6f};
  kda_prefill_plan_t plan;
  if (kda_abi_version() != KDA_ABI_VERSION) return 1;
  if (kda_prefill_plan(1, 8192, 8, -5.0f, 256, KDA_ROUTE_AUTO, &plan) != KDA_OK) return 2;
  if (plan.route != KDA_ROUTE_SPLIT || plan.windows < 3) return 3;
  /* invalid arguments are rejected on the host, before any device work */
  if (kda_decode_ex(0, 0, 0, 0, 0, 0, KDA_STATE_F32, 1, 0, 0, 1, 8, 128, 128, 1.0f, &fe, 0, 0)
      != KDA_ERR_INVALID_ARGUMENT) return 4;
  if (kda_last_error()[0] == '\0') return 5;
  printf("ok %d\n", (int)plan.windows);
  return 0;
}
''')
    lib_dir = os.path.dirname(kda.load()._name)
    exe = tmp_path / "use_kda"
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", str(src),
                        f"-L{lib_dir}", "-lkda", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout, r.stderr[-2000:])
