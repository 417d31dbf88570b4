"""Counter-based generator of bf16 test matrices (see the package docstring for the recipe)."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 20  # elements generated per numpy pass, bounds temporary memory


def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """SplitMix64 output for state ``seed + (c + 1) * GAMMA`` at each counter ``c`` (uint64)."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (c + np.uint64(1)) * GAMMA
        x = (x ^ (x >> np.uint64(30))) * _M1
        x = (x ^ (x >> np.uint64(27))) * _M2
        x = x ^ (x >> np.uint64(31))
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Used only to turn generated float32 samples into bf16 inputs. NaN is not produced by the
    generator, so no NaN special case is needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_chunk(seed: int, start: int, count: int, sigma: float) -> np.ndarray:
    idx = np.arange(start, start + count, dtype=np.uint64)
    r1 = splitmix64(seed, np.uint64(2) * idx)
    r2 = splitmix64(seed, np.uint64(2) * idx + np.uint64(1))
    u1 = ((r1 >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = (r2 >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return f32_to_bf16_bits((z * sigma).astype(np.float32))


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _chunked(count: int, fill) -> np.ndarray:
    """Run fill(offset, n) -> array over fixed chunks, in parallel threads (numpy drops the GIL)."""
    out = np.empty(count, dtype=np.uint16)
    starts = list(range(0, count, _CHUNK))

    def work(s):
        n = min(_CHUNK, count - s)
        out[s:s + n] = fill(s, n)

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, starts))
    return out


def normal_bf16(seed: int, count: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    """``count`` bf16 samples of N(0, sigma^2), elements ``start .. start+count-1`` of stream ``seed``."""
    return _chunked(count, lambda s, n: _normal_chunk(seed, start + s, n, sigma))


def integer_bf16(seed: int, count: int, radius: int = 4, start: int = 0) -> np.ndarray:
    """``count`` integers uniform-ish in [-radius, radius], as exact bf16 bit patterns."""
    if not (0 <= radius <= 128):
        raise ValueError("radius must be in [0, 128] so every value is exact in bf16")
    def fill(s, n):
        idx = np.arange(start + s, start + s + n, dtype=np.uint64)
        v = (splitmix64(seed, idx) >> np.uint64(32)) % np.uint64(2 * radius + 1)
        return f32_to_bf16_bits(v.astype(np.float32) - np.float32(radius))

    return _chunked(count, fill)


def ones_bf16(count: int) -> np.ndarray:
    return np.full(count, 0x3F80, dtype=np.uint16)


def matrix(kind: str, rows: int, cols: int, seed: int = 0, sigma: float = 1.0,
           radius: int = 4, ld: int | None = None) -> np.ndarray:
    """A rows x cols bf16 matrix (uint16 bits) in a row-major buffer with leading dimension ``ld``.

    ``kind`` is ``"normal"``, ``"int"`` or ``"ones"``. Padding columns (``ld > cols``) are filled
    with the bf16 pattern 0x7FC0 (a quiet NaN) so that a kernel reading them is caught.
    """
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld < cols")
    n = rows * cols
    if kind == "normal":
        flat = normal_bf16(seed, n, sigma)
    elif kind == "int":
        flat = integer_bf16(seed, n, radius)
    elif kind == "ones":
        flat = ones_bf16(n)
    else:
        raise ValueError(f"unknown kind {kind!r}")
    if ld == cols:
        return flat.reshape(rows, cols)
    out = np.full((rows, ld), 0x7FC0, dtype=np.uint16)
    out[:, :cols] = flat.reshape(rows, cols)
    return out
