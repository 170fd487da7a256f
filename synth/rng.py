"""Counter-based random inputs, bit-identical on the host (NumPy) and the device.

Every synthetic tensor element is a pure function of (stream key, counter), so
any slice of a tensor -- a slab of a 100M-token bank on the GPU, or the tokens
of a handful of sampled documents on the CPU -- can be regenerated anywhere
without generating the rest.

Generator
---------
* Mixing function: the SplitMix64 output finaliser (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
  z ^= z >> 31 (all arithmetic mod 2**64).
* Element ``n`` of stream ``key`` is ``mix64(key + (n + 1) * 0x9E3779B97F4A7C15)``,
  i.e. SplitMix64 seeded with ``key`` and advanced ``n + 1`` times.
* Approximately standard-normal values use the Irwin-Hall construction: the
  four 16-bit fields of the 64-bit output are summed (exact integer), centred,
  and scaled by one fp32 constant so that the variance is exactly 1:
  ``x = float32(2*s - 262140) * C``.  Integer work, one int->float conversion
  (exact below 2**24) and one IEEE fp32 multiply: bit-identical on every
  IEEE platform, which a transcendental Box-Muller step would not be.
  The law has mean 0, variance 1 and support |x| <= sqrt(12).
* Storage rounding: fp32 -> bfloat16 round-to-nearest-even on the bit pattern.

The device implementation of the same definition lives in
``synth/csrc/synth_gen.hip``.  This module contains no part of the method's
arithmetic: it only makes inputs.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
# 1 / (2 * sqrt((65536**2 - 1) / 3)) rounded to fp32 (0x1.bb67aep-17).
NORMAL_SCALE = np.float32(float.fromhex("0x1.bb67aep-17"))
_CENTRE = 262140  # 2 * (4 * 65535) / 2

ROLE_KR, ROLE_K, ROLE_V, ROLE_QR, ROLE_Q, ROLE_KLOC, ROLE_VLOC = range(7)
ROLE_SCORES = 7  # synthetic document scores for isolated top-k tests
ROLE_POOLED_KR, ROLE_POOLED_K, ROLE_POOLED_V = 8, 9, 10  # pooled-shape timing inputs
ROLE_HID_MEM, ROLE_HID_Q, ROLE_W_KR, ROLE_W_QR = 11, 12, 13, 14  # router-projector inputs


def _u64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.uint64)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    z = _u64(z)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, role: int, layer: int = 0) -> int:
    """Key of the stream for (seed, tensor role, layer): two chained mixes."""
    with np.errstate(over="ignore"):
        a = mix64(_u64([seed]) + GOLDEN * _u64([role + 1]))
        b = mix64(a + GOLDEN * _u64([layer + 1]))
    return int(b[0])


def raw_u64(key: int, counter0: int, n: int) -> np.ndarray:
    ctr = np.arange(n, dtype=np.uint64) + _u64(counter0 + 1)
    with np.errstate(over="ignore"):
        return mix64(_u64(key) + ctr * GOLDEN)


def normal_f32(key: int, counter0: int, n: int) -> np.ndarray:
    """n approximately-N(0,1) fp32 values of stream ``key`` from ``counter0``."""
    z = raw_u64(key, counter0, n)
    m = np.uint64(0xFFFF)
    s = (z & m) + ((z >> np.uint64(16)) & m) + ((z >> np.uint64(32)) & m) + (z >> np.uint64(48))
    c = (2 * s.astype(np.int64) - _CENTRE).astype(np.float32)
    return c * NORMAL_SCALE


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest, ties to even), returned as fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return b.astype(np.uint32).view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of fp32 values that are already bf16-representable."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable")
    return (b >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store_round(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage dtype ('f32' or 'bf16'); fp32 result."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


def normal_stored_numpy(key: int, counter0: int, n: int, dtype: str, block: int = 1 << 22) -> np.ndarray:
    """``store_round(normal_f32(...))`` in NumPy, in blocks to bound memory."""
    out = np.empty(n, dtype=np.float32)
    for a in range(0, n, block):
        b = min(n, a + block)
        out[a:b] = store_round(normal_f32(key, counter0 + a, b - a), dtype)
    return out


def normal_stored(key: int, counter0: int, n: int, dtype: str) -> np.ndarray:
    """Same values as ``normal_stored_numpy`` from the OpenMP C generator."""
    from . import native
    out = np.empty(n, dtype=np.float32)
    if n:
        native.host_lib().synth_normal(key, counter0, n, 1 if dtype == "bf16" else 0, out.ctypes.data)
    return out


def plant(x: np.ndarray, uhat: np.ndarray, cg: np.float32, dtype: str) -> np.ndarray:
    """Gold mixing of raw router keys: store_round(0.5*x + cg*uhat), in fp32.

    ``x`` is [..., H, d] of stored values, ``uhat`` is [H, d] fp32.  Two fp32
    roundings (product, sum) and the storage rounding, with no fused
    multiply-add, exactly as the device generator does.
    """
    x = np.asarray(x, dtype=np.float32)
    half = np.float32(0.5) * x
    prod = (np.float32(cg) * np.asarray(uhat, dtype=np.float32)).astype(np.float32)
    return store_round((half + prod).astype(np.float32), dtype)


def plant_fast(x: np.ndarray, uhat: np.ndarray, cg: np.float32, dtype: str) -> np.ndarray:
    """``plant`` on a contiguous [n][H][d] fp32 array, in place, by the C generator."""
    from . import native
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = np.ascontiguousarray(uhat, dtype=np.float32)
    native.host_lib().synth_plant(x.ctypes.data, x.shape[0], x.shape[1], x.shape[2], u.ctypes.data,
                                  float(cg), 1 if dtype == "bf16" else 0)
    return x
