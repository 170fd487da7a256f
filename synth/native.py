"""Build and load the two native input generators (host C + OpenMP, device HIP).

``build()`` always compiles; ``host_lib()`` / ``dev_lib()`` load what is built
and compile only when nothing is.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

_HERE = Path(__file__).resolve().parent
HOST_SO = _HERE / "libmsa_synth_host.so"
DEV_SO = _HERE / "libmsa_synth_dev.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

_host = None
_dev = None


def build_host() -> Path:
    src = _HERE / "csrc" / "synth_host.c"
    tmp = HOST_SO.with_suffix(".so.tmp")
    subprocess.run(["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", str(src), "-o", str(tmp)],
                   check=True)
    os.replace(tmp, HOST_SO)
    return HOST_SO


def build_dev() -> Path:
    src = _HERE / "csrc" / "synth_gen.hip"
    tmp = DEV_SO.with_suffix(".so.tmp")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    str(src), "-o", str(tmp)], check=True, stderr=subprocess.DEVNULL)
    os.replace(tmp, DEV_SO)
    return DEV_SO


def build() -> None:
    build_host()
    build_dev()


def host_lib():
    global _host
    if _host is None:
        if not HOST_SO.exists():
            build_host()
        lib = ctypes.CDLL(str(HOST_SO))
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        lib.synth_normal.restype = None
        lib.synth_normal_bf16_bits.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_normal_bf16_bits.restype = None
        lib.synth_plant.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_float, ctypes.c_int]
        lib.synth_plant.restype = None
        _host = lib
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime, loaded first)
        if not DEV_SO.exists():
            build_dev()
        lib = ctypes.CDLL(str(DEV_SO))
        lib.synth_dev_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                              ctypes.c_int, ctypes.c_void_p]
        lib.synth_dev_fill_normal.restype = ctypes.c_int
        lib.synth_dev_plant.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.synth_dev_plant.restype = ctypes.c_int
        _dev = lib
    return _dev
