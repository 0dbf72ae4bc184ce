"""Build the gfx950 HIP library in-tree: mla_decode_attention_amd/libmla_decode.so."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-FP32 VALU ops stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in arch VGPRs: the online-softmax rescale multiplies them with
    # VALU ops, which cannot address AGPRs (AGPR accumulators cost a copy per tile)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# translation units of the library and whether each keeps the arch-VGPR accumulator option
UNITS = [("mla_decode.hip", True)]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None,
          csrc: str | None = None) -> str:
    """Compile every translation unit to an object, then link the shared library.  extra_flags go
    to every compile; csrc replaces the source folder (for builds of modified copies)."""
    out = out or LIB
    src = csrc or CSRC
    tag = f"{os.getpid()}"
    objs = []
    compile_flags = [f for f in FLAGS if f != "-shared"]
    compile_flags = [src if f == CSRC else f for f in compile_flags]
    try:
        for name, vgpr_form in UNITS:
            obj = f"{out}.{name}.{tag}.o"
            fl = compile_flags if vgpr_form else [f for f in compile_flags
                                                  if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form=1")]
            _run([HIPCC, *fl, *(extra_flags or []), "-c", os.path.join(src, name), "-o", obj], verbose)
            objs.append(obj)
        tmp = f"{out}.tmp{tag}"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(tmp, out)
    return out


PROBE_LIB = os.path.join(PKG, "libmla_read_probe.so")


def build_read_probe(verbose: bool = False) -> str:
    """The streaming-read probe bench.py times beside the decode kernels (its own library)."""
    tmp = f"{PROBE_LIB}.tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, os.path.join(CSRC, "read_probe.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose:
        print(" ".join(cmd), flush=True)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
