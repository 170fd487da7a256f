"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): libmsa.so is rebuilt with host-only sanitizer instrumentation
(the device code is compiled as usual) into _build/sanitize/, loaded by a
copy of the binding in a scratch directory, and tests/test_abi.py runs against
it in a child process with the sanitizer runtime preloaded.  Any report
(out-of-bounds access, use after free, undefined behaviour) fails the run."""
import importlib.util
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
PKG = "long_context_memory_msa_amd"


def _asan_runtime() -> str:
    clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    return path


@pytest.mark.slow
def test_abi_validation_under_host_sanitizers(tmp_path):
    spec = importlib.util.spec_from_file_location("_msa_build_sanitize", ROOT / PKG / "build.py")
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    lib = build.build(sanitize=True)
    undef = subprocess.run(["nm", "-D", "--undefined-only", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_report_load8" in undef and "__ubsan_handle" in undef, "library is not instrumented"
    # a scratch tree: the binding next to the sanitized library, the ABI tests, the header they read
    (tmp_path / PKG).mkdir()
    for f in (ROOT / PKG).glob("*.py"):
        shutil.copy(f, tmp_path / PKG / f.name)
    shutil.copy(lib, tmp_path / PKG / "libmsa.so")
    (tmp_path / "tests").mkdir()
    for f in ("test_abi.py", "conftest.py"):
        shutil.copy(ROOT / "tests" / f, tmp_path / "tests" / f)
    (tmp_path / "include").mkdir()
    shutil.copy(ROOT / "include" / "msa.h", tmp_path / "include" / "msa.h")
    shutil.copy(ROOT / "pytest.ini", tmp_path / "pytest.ini")
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = (f"import {PKG}._lib as L, pathlib; "
             f"assert pathlib.Path(L.LIB_PATH).resolve() == pathlib.Path({str(tmp_path / PKG / 'libmsa.so')!r}); "
             "print('sanitized library loaded')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=tmp_path, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "sanitized library loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"],
                       cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
