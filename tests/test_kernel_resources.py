"""Register, scratch and occupancy budget of the gfx950 kernels (CPU only).

Each source is compiled for the device with the flags the library build
uses plus the compiler's resource-usage remarks.  No kernel may use scratch
memory (a spill would put per-lane private memory traffic on the hot path),
and the split-route kernels must keep two waves per SIMD: the chain planner
sizes its windows for two chain blocks per compute unit, and the preparation
pass relies on two waves per SIMD to keep enough loads in flight.
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
