"""Build libattn.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled on each call (objects go to ``_build/`` at the
repository root) and linked into ``transformer_attention_split_amd/libattn.so``.
Run as ``python transformer_attention_split_amd/build.py`` (by path, so that
the package, which loads the library on import, is not imported first);
``--sanitize`` builds the host-sanitized test library of the C ABI layer
instead (``_build/san/libattn_san.so``).
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


# Host-side sanitizers for the C ABI layer (argument checks, planning,
# error reporting): api.cpp is compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host pass only (each -fsanitize= follows
# -Xarch_host; the device code is built as usual) and linked with the normal
# kernel objects into a separate test library. Loading it needs the ASan
# runtime preloaded (asan_runtime()).
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libattn_san.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The shared ASan runtime of the HIP toolchain's clang."""
    hipcc = os.path.realpath(_hipcc())
    roots = [os.path.join(os.path.dirname(os.path.dirname(hipcc)), "llvm"),
             "/opt/rocm/llvm"]
    for root in roots:
        base = os.path.join(root, "lib", "clang")
        if not os.path.isdir(base):
            continue
        for ver in sorted(os.listdir(base), reverse=True):
            cand = os.path.join(base, ver, "lib", "linux",
                                "libclang_rt.asan-x86_64.so")
            if os.path.exists(cand):
                return cand
    raise RuntimeError("libclang_rt.asan-x86_64.so not found")


def build_sanitized(verbose: bool = False) -> str:
    """Build SAN_LIB: api.cpp with host ASan + UBSan, kernels as in build()."""
    build(verbose=verbose)  # kernel objects in BUILD
    hipcc = _hipcc()
    os.makedirs(SAN_DIR, exist_ok=True)
    api_o = os.path.join(SAN_DIR, "api.o")
    cmd = [hipcc, *HIPFLAGS, "-O1", "-g", *SAN_HOST_FLAGS, "-x", "hip", "-c",
           os.path.join(CSRC, "api.cpp"), "-o", api_o]
    rc, out = _run(cmd)
    if verbose or rc != 0:
        print(out, file=sys.stderr)
    if rc != 0:
        raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}")
    objs = [api_o] + [os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
                      for src in SOURCES if src != "api.cpp"]
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared",
                    "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
                    "-o", SAN_LIB, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link of the sanitized library failed")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
