"""Chunk-seeded random number generation and bf16 storage helpers.

Every tensor is drawn in fixed-size chunks; chunk c of tensor `tag` under seed `s`
uses its own PCG64 stream seeded from SeedSequence([s, tag, c]). The result is
therefore identical whatever the number of threads used to fill it.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, tag: int, n: int, std: float = 1.0) -> np.ndarray:
    """n draws of N(0, std^2) in float32 (std applied in float32)."""
    out = np.empty(n, dtype=np.float32)

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, c])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def normal_f32_range(seed: int, tag: int, lo: int, hi: int, std: float = 1.0) -> np.ndarray:
    """Elements lo .. hi-1 of normal_f32(seed, tag, n, std), for any n >= hi: each chunk's
    stream is drawn from its start, and a shorter draw is a prefix of a longer one."""
    out = np.empty(max(0, hi - lo), dtype=np.float32)
    if hi <= lo:
        return out

    def fill(c: int) -> None:
        a = max(lo, c * CHUNK)
        b = min(hi, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, c])))
        buf = g.standard_normal(b - c * CHUNK, dtype=np.float32)
        out[a - lo:b - lo] = buf[a - c * CHUNK:]
        if std != 1.0:
            out[a - lo:b - lo] *= np.float32(std)

    chunks = range(lo // CHUNK, (hi - 1) // CHUNK + 1)
    if len(chunks) <= 1:
        for c in chunks:
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, chunks))
    return out


def rng(seed: int, tag: int) -> np.random.Generator:
    """A small-draw generator (positions, lengths) for one purpose of one seed."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, 1 << 30])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bfloat16 bit patterns as uint16. Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = CHUNK

    def conv(lo: int) -> None:
        hi = min(u.size, lo + step)
        a = u.reshape(-1)[lo:hi].astype(np.uint64)
        a = (a + 0x7FFF + ((a >> 16) & 1)) >> 16
        out.reshape(-1)[lo:hi] = a.astype(np.uint16)

    starts = range(0, u.size, step)
    if u.size <= step:
        for lo in starts:
            conv(lo)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, starts))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3_encode(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes of x / scale in OCP FP8 E4M3 (round to nearest, ties to even), saturated at
    +-448, the largest finite value; returned as uint8. Inputs must be finite. The
    rounding is torch's float32 -> float8_e4m3fn conversion."""
    import torch

    y = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) / float(scale)
    y.clamp_(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def stored_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen stored values (bf16 bit patterns as uint16, or float32) to float64 exactly."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError(f"unexpected stored dtype {a.dtype}")
