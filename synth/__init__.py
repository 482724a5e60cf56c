"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no arithmetic of the compressed-attention method: it draws
random bits and random floats, and writes cache images directly as random
codes (never through a quantizer).  Both the oracle and the HIP path consume
what it returns; neither is imported here.

Generator: counter-based SplitMix64.  Element i of a stream with key K is
mix(K + (i + 1) * 0x9E3779B97F4A7C15), where mix is the SplitMix64 output
function (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014).  Stream keys come from (seed, tensor name, row ...)
through the same function, so any slice of any stream can be regenerated on
its own: a full-size parity test regenerates only the rows it samples.
Normals use the Box-Muller transform on consecutive pairs of uniforms.
"""
from __future__ import annotations

import zlib

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1


def _mix_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def _mix(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def key(seed: int, *ids) -> int:
    """Stream key for (seed, ids...); ids may be ints or strings."""
    k = _mix_int(int(seed) * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019)
    for x in ids:
        v = zlib.crc32(x.encode()) if isinstance(x, str) else int(x)
        k = _mix_int(k ^ _mix_int(v + 0x9E3779B97F4A7C15))
    return k


def u64(k: int, n: int, offset: int = 0) -> np.ndarray:
    with np.errstate(over="ignore"):
        i = np.arange(offset + 1, offset + 1 + n, dtype=np.uint64)
        return _mix(np.uint64(k) + i * GOLDEN)


def uniform(k: int, n: int, offset: int = 0) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (u64(k, n, offset) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(k: int, n: int, offset: int = 0) -> np.ndarray:
    """N(0, 1) doubles; element i uses uniforms 2*i and 2*i + 1 of the stream."""
    u = uniform(k, 2 * n, 2 * offset).reshape(n, 2)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
    return r * np.cos(2.0 * np.pi * u[:, 1])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """A random bf16 value from a random float: the top half of its fp32 bits."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def randbytes(k: int, n: int) -> np.ndarray:
    words = u64(k, (n + 7) // 8)
    return words.view(np.uint8)[:n].copy()


# ---------------------------------------------------------------------------
# Tensors of the workloads
# ---------------------------------------------------------------------------

def normal_f32(seed, name, shape, *ids) -> np.ndarray:
    n = int(np.prod(shape))
    return normal(key(seed, name, *ids), n).astype(np.float32).reshape(shape)


def abs_normal_f32(seed, name, shape, *ids) -> np.ndarray:
    return np.abs(normal_f32(seed, name, shape, *ids))


def bf16_normal(seed, name, shape, *ids) -> np.ndarray:
    return bf16_bits(normal_f32(seed, name, shape, *ids))


def e4m3_code_image(seed, name, n, *ids) -> np.ndarray:
    """Random FP8 e4m3fn codes: a random byte, the two NaN codes moved to +-448."""
    b = randbytes(key(seed, name, *ids), n)
    b[(b & 0x7F) == 0x7F] -= 1
    return b


def fp8_scale_image(seed, name, n, *ids) -> np.ndarray:
    """Per-64 fp32 scales uniform in [2/448, 3/448] (the range an amax/448 scale
    takes for N(0,1) groups)."""
    u = uniform(key(seed, name, *ids), n)
    return ((2.0 + u) / 448.0).astype(np.float32)


def e2m1_code_image(seed, name, n_bytes, *ids) -> np.ndarray:
    """Random packed FP4 e2m1 code bytes (every nibble is a valid code)."""
    return randbytes(key(seed, name, *ids), n_bytes)


def e8m0_image(seed, name, n, *ids) -> np.ndarray:
    """E8M0 block exponents 2^-3 .. 2^0."""
    return (127 - (u64(key(seed, name, *ids), n) % np.uint64(4))).astype(np.uint8)


def distinct_choice(seed, name, count, lo, hi, *ids) -> np.ndarray:
    """`count` distinct integers drawn uniformly from [lo, hi] (sorted)."""
    span = hi - lo + 1
    if count > span:
        raise ValueError("not enough distinct values")
    chosen = []
    seen = set()
    i = 0
    k = key(seed, name, *ids)
    while len(chosen) < count:
        v = lo + int(u64(k, 1, i)[0] % np.uint64(span))
        i += 1
        if v not in seen:
            seen.add(v)
            chosen.append(v)
    return np.array(sorted(chosen), dtype=np.int64)
