"""The C ABI layer under host AddressSanitizer + UndefinedBehaviorSanitizer
(CPU only): build the sanitized test library (api.cpp instrumented on its
host pass, kernels as usual) and run the whole of tests/test_abi.py against
it in a fresh interpreter with the ASan runtime preloaded. Any sanitizer
report aborts that run (halt_on_error), so a clean exit means every argument
check, error path and status string of the ABI ran free of memory errors and
undefined behaviour."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.slow


def _build_script():
    """The package's build script, loaded by path (importing the package
    would load the library it builds)."""
    path = os.path.join(ROOT, "transformer_attention_split_amd", "build.py")
    spec = importlib.util.spec_from_file_location("attn_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    build = _build_script()
    try:
        runtime = build.asan_runtime()
    except RuntimeError as exc:
        pytest.skip(str(exc))
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update(
        ATTN_LIB_PATH=lib,
        LD_PRELOAD=runtime,
        ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:"
                     f"log_path={tmp_path}/asan",
        UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan",
    )
    p = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
         "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(os.listdir(tmp_path))
    detail = "".join(open(os.path.join(tmp_path, r)).read() for r in reports)
    assert p.returncode == 0 and not reports, (p.stdout[-2000:], detail[:4000])
    assert " passed" in p.stdout
