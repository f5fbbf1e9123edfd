"""Counter-based random numbers for the seeded synthetic workloads (host side).

This module holds no arithmetic of the attention method: it only turns
(seed, tensor id, element index) into bits.  The device fill kernels in
``synth/fill.hip`` implement the very same definitions, so any slice of a
device tensor can be regenerated here bit for bit.

Definitions
-----------
* ``mix64`` is the SplitMix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014): xor-shift
  by 30, multiply by 0xBF58476D1CE4E5B9, xor-shift by 27, multiply by
  0x94D049BB133111EB, xor-shift by 31, all modulo 2**64.
* A stream is named by ``key = mix64(seed XOR (tensor_id * GAMMA))`` with
  ``GAMMA = 0x9E3779B97F4A7C15``; its n-th 64-bit word is
  ``mix64(key + (n + 1) * GAMMA)``, i.e. SplitMix64 started at state ``key``
  and evaluated out of order.
* ``normal`` element i: words 2i and 2i+1 give eight 16-bit unsigned lanes;
  their sum s (an Irwin-Hall variate of order 8) is centred and scaled as
  ``float32(2*s - 524280) * NORMAL_SCALE`` (one float32 rounding), then
  rounded to bfloat16 with round-to-nearest-even.  Mean 0, variance 1,
  support +-4.9.  Integer arithmetic up to the single float32 multiply makes
  host and device agree bit for bit.
* ``small_int`` element i: ``((word_i >> 48) % 5) - 2``, a value in
  {-2,...,2}, stored exactly in bfloat16.  Dot products of such vectors are
  exact in float32, which the exact-parity tests rely on.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB

# 1 / (2 * sqrt(8 * (65536**2 - 1) / 12)), rounded to float32 once and fixed
# here by its bit pattern so that both sides use the identical constant.
NORMAL_SCALE_BITS = 0x371CC471
NORMAL_SCALE = np.uint32(NORMAL_SCALE_BITS).view(np.float32)

_U64 = np.uint64


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX_M1) & MASK64
    z = ((z ^ (z >> 27)) * MIX_M2) & MASK64
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function, element-wise on a uint64 array."""
    z = z.astype(_U64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> _U64(30)
        z *= _U64(MIX_M1)
        z ^= z >> _U64(27)
        z *= _U64(MIX_M2)
        z ^= z >> _U64(31)
    return z


def stream_key(seed: int, tensor_id: int) -> int:
    """Key of the stream named by (seed, tensor_id)."""
    return mix64_int((seed ^ ((tensor_id * GAMMA) & MASK64)) & MASK64)


def words(key: int, n: np.ndarray) -> np.ndarray:
    """The n-th 64-bit words of stream ``key`` (n: integer array)."""
    n = np.asarray(n, dtype=_U64)
    with np.errstate(over="ignore"):
        state = _U64(key) + (n + _U64(1)) * _U64(GAMMA)
    return mix64(state)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bits, nearest-even (inputs are finite)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(key: int, idx: np.ndarray) -> np.ndarray:
    """bfloat16 bits of the ``normal`` variate for element indices ``idx``."""
    idx = np.asarray(idx, dtype=_U64)
    w0 = words(key, idx * _U64(2))
    w1 = words(key, idx * _U64(2) + _U64(1))
    s = np.zeros(idx.shape, dtype=np.int64)
    mask = _U64(0xFFFF)
    for w in (w0, w1):
        for sh in (0, 16, 32, 48):
            s += ((w >> _U64(sh)) & mask).astype(np.int64)
    x = (2 * s - 524280).astype(np.int32).astype(np.float32)
    return f32_to_bf16_bits(x * NORMAL_SCALE)


def small_int_bf16(key: int, idx: np.ndarray) -> np.ndarray:
    """bfloat16 bits of the ``small_int`` variate (values -2..2)."""
    w = words(key, np.asarray(idx, dtype=_U64))
    v = ((w >> _U64(48)) % _U64(5)).astype(np.int32) - 2
    return f32_to_bf16_bits(v.astype(np.float32))


def draw_ints(key: int, start: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` integers in [lo, hi) from words start.. of stream ``key``.

    Uses ``lo + word % (hi - lo)``; the modulo bias is below 2**-40 for the
    ranges used here.
    """
    w = words(key, np.arange(start, start + count, dtype=_U64))
    return (w % _U64(hi - lo)).astype(np.int64) + lo


def permutation(key: int, n: int) -> np.ndarray:
    """Seeded permutation of range(n): argsort of n stream words (ties by index)."""
    w = words(key, np.arange(n, dtype=_U64))
    return np.argsort(w, kind="stable").astype(np.int64)
