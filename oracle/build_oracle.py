"""Compile the fp64 CPU oracle (test infrastructure) into a shared library next to this file."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mla_oracle.c")


def lib_path(planted_mistake: int = 0) -> str:
    name = "libmla_oracle.so" if planted_mistake == 0 else f"libmla_oracle_planted{planted_mistake}.so"
    return os.path.join(HERE, name)


def build(planted_mistake: int = 0, out: str | None = None) -> str:
    """gcc -O2 -fopenmp; planted_mistake > 0 builds a deliberately wrong variant for pin tests."""
    out = out or lib_path(planted_mistake)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           f"-DORACLE_PLANTED_MISTAKE={int(planted_mistake)}", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0))
