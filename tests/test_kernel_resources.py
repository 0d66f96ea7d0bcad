"""Register, scratch and occupancy budget of the gfx950 kernels (CPU only).

Each source is compiled for the device with the flags the library build
uses plus the compiler's resource-usage remarks.  No kernel may use scratch
memory (a spill would put per-lane private memory traffic on the hot path),
and the split-route kernels must keep two waves per SIMD: the chain planner
sizes its windows for two chain blocks per compute unit, and the preparation
pass relies on two waves per SIMD to keep enough loads in flight.

The generated code is also scanned for a 12- or 16-byte vector-memory store
followed, with no wait state between, by a VALU write to the store's data
registers: the hardware may still be reading them, and the compiler omits
that wait state for buffer stores whose offset is held in an SGPR (a decode
kernel built that way wrote corrupted state words).
"""
import os
import re
import shutil
import subprocess

import pytest

from kimi_delta_attention_prefill_amd import build as kbuild

MIN_WAVES = {
    "prefill_split_prep": 2,
    "prefill_split_chain": 2,
    "prefill_split_window_a": 2,
    "prefill_split_window_c": 2,
    # the many-row decode shapes: three 512-thread blocks (three whole-item
    # state streams) resident per compute unit
    "decode_kernelILi128ELb0ELi512E": 6,
    "decode_kernelILi128ELb1ELi512E": 6,
}


def _resources(src):
    cmd = ([kbuild.hipcc(), "-x", "hip"] + kbuild._flags() + kbuild._EXTRA.get(os.path.basename(src), [])
           + ["-Rpass-analysis=kernel-resource-usage", "--offload-device-only", "-c", src,
              "-o", os.devnull])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split(" ")[0]] = int(m.group(2))
    return kernels


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is not available")
@pytest.mark.parametrize("source", ["prefill_split.hip", "prefill_chunk.hip", "prefill_serial.hip",
                                    "decode.hip"])
def test_no_scratch_and_occupancy(source):
    kernels = _resources(os.path.join(kbuild.CSRC, source))
    assert kernels, "no kernel resource remarks"
    for name, res in kernels.items():
        assert res.get("ScratchSize", 0) == 0, f"{name} spills: {res}"
        for short, waves in MIN_WAVES.items():
            if short in name:
                assert res["Occupancy"] >= waves, f"{name}: {res}"


def _asm(src):
    cmd = ([kbuild.hipcc(), "-x", "hip"] + kbuild._flags() + kbuild._EXTRA.get(os.path.basename(src), [])
           + ["--offload-device-only", "-S", src, "-o", "-"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return [ln.strip() for ln in r.stdout.splitlines()
            if ln.strip() and not ln.strip().startswith((";", "."))]


def _vregs(spec):
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is not available")
@pytest.mark.parametrize("source", ["prefill_split.hip", "prefill_chunk.hip", "prefill_serial.hip",
                                    "decode.hip", "check.hip"])
def test_no_wide_store_data_overwrite(source):
    lines = _asm(os.path.join(kbuild.CSRC, source))
    stores = 0
    for i, ln in enumerate(lines):
        m = re.match(r"(global|buffer|flat)_store_dword(x3|x4)\s+(\S+?),\s*(\S+?)(,|\s|$)", ln)
        if not m:
            continue
        stores += 1
        data = _vregs(m.group(4) if m.group(1) in ("global", "flat") else m.group(3))
        for nxt in lines[i + 1:i + 3]:
            if nxt.startswith("s_nop") or not nxt.startswith("v_"):
                break
            dst = nxt.split()[1].rstrip(",")
            assert not (_vregs(dst) & data), f"{source}: '{ln}' then '{nxt}'"
