"""Build step for the CPU oracle: gcc, IEEE binary32, no FMA contraction."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "nf4_oracle.c")
OUT = os.path.join(_HERE, "libnf4_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build_oracle(force: bool = True) -> str:
    if not force and os.path.exists(OUT) and os.path.getmtime(OUT) >= os.path.getmtime(SRC):
        return OUT
    tmp = OUT + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm", "-lpthread"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_oracle())
