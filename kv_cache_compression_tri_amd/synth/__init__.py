"""Seeded synthetic inputs for the compression pass (test and benchmark infrastructure).

This module holds no step of the compression method.  It defines one counter-based
generator of key/value elements, implemented twice from the same published definitions:
here in numpy (host, for the oracle's inputs and small cases) and in ``csrc/synth.hip``
(device, for the full-size caches).  Both produce bit-identical values:

* hash:   SplitMix64's output function ``mix64`` (Steele, Lea & Flood, "Fast splittable
          pseudorandom number generators", OOPSLA 2014), applied to the counter
          ``key + n * 0x9E3779B97F4A7C15`` (the SplitMix64 stream read at index n).
* normal: Irwin-Hall sum of twelve 16-bit uniforms minus 6 (a classic N(0, 1)
          approximation with unit variance), formed as an exact integer numerator times
          2^-16, so it is exact in float32.
* value:  ``x = mu[col] + sigma[col] * n`` in float32 with each operation rounded once
          (no fused multiply-add), times 20 on a sink row, then rounded to bfloat16 with
          round-to-nearest-even, kept as float32, or (fp8, int8) multiplied by a power-of-two
          inverse scale and encoded as OCP E4M3 (round to nearest even, saturating at 448)
          or as int8 (round to nearest even, clamped to [-127, 127]).

Element (unit, row, col) of stream ``tag`` under ``seed`` uses counter
``c = unit << 27 | row << 7 | col`` (row < 2^20, col < 128) and the three hashes at
SplitMix64 indices 3c+1, 3c+2, 3c+3 of the stream keyed by ``mix64(seed << 8 | tag)``.
"""

from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_U64 = np.uint64

TAG_K = 0
TAG_V = 1
SINK_SCALE = np.float32(20.0)
MAX_ROWS = 1 << 20


def mix64(z):
    """SplitMix64 output function on uint64 arrays (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> _U64(30))) * _M1
    z = (z ^ (z >> _U64(27))) * _M2
    return z ^ (z >> _U64(31))


def stream_key(seed: int, tag: int) -> np.uint64:
    if not (0 <= seed < (1 << 56)) or not (0 <= tag < 256):
        raise ValueError("seed must be in [0, 2^56) and tag in [0, 256)")
    return mix64(np.array([(seed << 8) | tag], dtype=np.uint64))[0]


def normals(seed: int, tag: int, unit: int, rows, cols=128) -> np.ndarray:
    """Irwin-Hall(12) - 6 variates for element counters (unit, rows[i], col), float32 [R, cols]."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    col = np.arange(cols, dtype=np.uint64).reshape(1, -1)
    if rows.size and int(rows.max()) >= MAX_ROWS:
        raise ValueError("row index out of the counter's range")
    c = (_U64(unit) << _U64(27)) | (rows << _U64(7)) | col
    key = stream_key(seed, tag)
    s = np.zeros(c.shape, dtype=np.int64)
    with np.errstate(over="ignore"):
        for i in range(3):
            h = mix64(key + (_U64(3) * c + _U64(i + 1)) * _U64(GAMMA))
            for w in range(4):
                s += ((h >> _U64(16 * w)) & _U64(0xFFFF)).astype(np.int64)
    m = (s - 393210).astype(np.float32)
    return m * np.float32(2.0 ** -16)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_fp8_e4m3(x) -> np.ndarray:
    """OCP E4M3 codes of float32 values: round to nearest even on the float32 bits,
    subnormal steps of 2^-9 below 2^-6, saturation at +-448, NaN -> S.1111.111."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.int64)
    sign = (u >> 24) & 0x80
    a = u & 0x7FFFFFFF
    e0 = (a >> 23) - 127
    r = (a >> 20) & 7
    rem = a & 0xFFFFF
    r = r + ((rem > 0x80000) | ((rem == 0x80000) & ((r & 1) == 1))).astype(np.int64)
    carry = r == 8
    r = np.where(carry, 0, r)
    e = e0 + carry
    normal = np.where(e > 8, 0x7E, ((e + 7) << 3) | r)
    normal = np.minimum(normal, 0x7E)
    with np.errstate(over="ignore", invalid="ignore"):
        sub = np.rint(np.abs(x) * np.float32(512.0)).astype(np.float64)
    sub = np.where(e0 < -6, sub, 0).astype(np.int64)
    code = np.where(e0 >= -6, normal, sub)
    code = np.where(a > 0x7F800000, 0x7F, code)
    return (sign | code).astype(np.uint8)


def f32_to_int8(x) -> np.ndarray:
    """Symmetric int8 codes of float32 values: round to nearest even, clamp to [-127, 127]."""
    x = np.asarray(x, dtype=np.float32)
    return np.clip(np.rint(x), -127, 127).astype(np.int8)


def rows(seed: int, tag: int, unit: int, n_rows: int, mu, sigma, sink: bool,
         dtype: str = "bf16", row_start: int = 0, scale: float = 1.0) -> np.ndarray:
    """Rows row_start .. row_start+n_rows-1 of one unit.

    Returns float32 [n_rows, 128] for dtype "f32", uint16 bfloat16 bits for "bf16",
    uint8 E4M3 codes of x / scale for "fp8" and int8 codes of x / scale for "int8" (scale a
    power of two, so x / scale is exact before rounding).
    """
    r = np.arange(row_start, row_start + n_rows, dtype=np.uint64)
    n = normals(seed, tag, unit, r, len(mu))
    mu = np.asarray(mu, dtype=np.float32)[None, :]
    sigma = np.asarray(sigma, dtype=np.float32)[None, :]
    x = mu + sigma * n                       # two float32 roundings, as on the device
    if sink and row_start == 0 and n_rows > 0:
        x[0] = SINK_SCALE * x[0]
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp8":
        return f32_to_fp8_e4m3(x * np.float32(1.0 / scale))
    if dtype == "int8":
        return f32_to_int8(x * np.float32(1.0 / scale))
    raise ValueError(f"unknown dtype {dtype!r}")
