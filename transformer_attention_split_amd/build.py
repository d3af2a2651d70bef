"""Build libattn.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled on each call (objects go to ``_build/`` at the
repository root) and linked into ``transformer_attention_split_amd/libattn.so``.
Run as ``python transformer_attention_split_amd/build.py`` (by path, so that
the package, which loads the library on import, is not imported first).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")

ARCH = "gfx950"
SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "topk.hip", "probe.hip"]

# Per-source extra flags. The prefill kernel never lets a NaN reach its
# arithmetic (rows past the valid length are not read; -inf is used for
# masking and stays supported), so it is compiled with NaNs assumed absent
# and the IEEE mode bit off: fmax then needs no operand quieting.
SOURCE_FLAGS = {"prefill.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}

# Packed fp32 VALU forms are disabled; the host pass warns that it does not
# know the feature, which is harmless.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"),
                 "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "packed-fp32-ops" not in line)
    return p.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmds.append([hipcc, *HIPFLAGS, *SOURCE_FLAGS.get(src, []), *lang,
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            if out.strip():
                print(out, file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}")
    tmp = LIB + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-o", tmp,
                    *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link of libattn.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
