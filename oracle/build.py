"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(force: bool = True) -> str:
    out = os.path.join(_HERE, "liboracle.so")
    src = os.path.join(_HERE, "oracle.c")
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wextra", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", src, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
