"""Compile the plain C client of the library (test infrastructure) next to this file.

gcc builds it against the HIP runtime's C API (the platform macro selects the AMD headers for a
non-HIP compiler) and links libmla_decode.so from the package directory (rpath relative to the
binary, so the tree can move)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_from_c.c")
BIN = os.path.join(HERE, "decode_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = f"{BIN}.tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "mla_decode_attention_amd"), "-lmla_decode",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../mla_decode_attention_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
