"""Compile libmsa.so (all HIP kernels + the C ABI) for gfx950, in-tree.

``build()`` always recompiles; the binding calls it only when no library is
present.  Objects go to ``_build/`` (not committed); the shared library is
written next to this file.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

HERE = Path(__file__).resolve().parent
CSRC = HERE / "csrc"
ROOT = HERE.parent
LIB = HERE / "libmsa.so"
OBJ_DIR = ROOT / "_build" / "msa"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.cpp", "pool.hip", "route.hip", "route_wide.hip", "topk.hip", "attend.hip", "project.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # never emit packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}",
]


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer build (the device
# code is compiled as usual): for the ABI's host-side validation, run on the
# CPU with the sanitizer runtime preloaded.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SANITIZE_DIR = ROOT / "_build" / "sanitize"


def _compile(src: str, obj_dir: Path, extra: list) -> Path:
    obj = obj_dir / (src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> Path:
    """Compile and link libmsa.so; ``sanitize`` builds the host-sanitized
    variant into _build/sanitize/ instead (never loaded by the package)."""
    obj_dir = SANITIZE_DIR / "obj" if sanitize else OBJ_DIR
    lib = SANITIZE_DIR / "libmsa.so" if sanitize else LIB
    extra = SANITIZE_FLAGS if sanitize else []
    obj_dir.mkdir(parents=True, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, extra), SOURCES))
    tmp = lib.with_suffix(".so.tmp")
    # --no-undefined: a kernel whose host stub was not emitted fails here, not at load time
    # (the sanitized variant leaves the sanitizer runtime to the preloaded library)
    link = ["-shared-libasan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] \
        if sanitize else ["-Wl,--no-undefined"]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {lib.name} failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
