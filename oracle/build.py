"""Build the FP64 oracle shared library with the host C compiler (test infrastructure)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile ``kda_oracle.c`` into ``liboracle.so`` (plain C, -O2, no fast-math)."""
    src = os.path.join(_HERE, "kda_oracle.c")
    out = library_path()
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
