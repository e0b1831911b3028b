"""Seeded, tensor-keyed random streams for synthetic inputs.

Every tensor is drawn from its own stream, keyed by (seed, crc32(name), block),
so any tensor (or any 2**22-element block of it) can be regenerated on its own
and the result does not depend on how many threads draw it.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, name: str, block: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), zlib.crc32(name.encode()), block]))


def _fill(n: int, draw):
    """Fill n values block by block (in parallel); draw(block_index, count) -> array."""
    nblk = (n + BLOCK - 1) // BLOCK
    out = np.empty(n, np.float32)

    def one(j):
        lo = j * BLOCK
        cnt = min(BLOCK, n - lo)
        out[lo:lo + cnt] = draw(j, cnt)

    if nblk <= 1:
        for j in range(nblk):
            one(j)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(one, range(nblk)))
    return out


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x32, np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal(seed, name, shape, std=1.0, mean=None, dtype="f32"):
    """N(0, std^2) values (plus an optional float32 array ``mean`` of the same shape)
    stored as float32 (dtype "f32") or bf16 bit patterns (dtype "bf16")."""
    n = int(np.prod(shape))
    std32 = np.float32(std)

    def draw(j, cnt):
        v = _rng(seed, name, j).standard_normal(cnt, dtype=np.float32)
        v *= std32
        return v

    x = _fill(n, draw).reshape(shape)
    if mean is not None:
        x += np.asarray(mean, np.float32).reshape(shape)
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def uniform01(seed, name, shape):
    """U[0,1) drawn in float64, rounded to float32 and kept strictly below 1."""
    n = int(np.prod(shape))
    u = _rng(seed, name).random(n).astype(np.float32)
    u = np.minimum(u, np.float32(1.0) - np.float32(2.0 ** -24))
    return u.reshape(shape)


def integers(seed, name, shape, low, high):
    return _rng(seed, name).integers(low, high, size=shape).astype(np.int32)


def gains(seed, name, n, std, dtype):
    """Norm gains 1 + N(0, std^2) (exactly 1 when std == 0)."""
    g = np.ones(n, np.float32)
    if std > 0:
        g += normal(seed, name, (n,), std, dtype="f32")
    return to_bf16_bits(g) if dtype == "bf16" else g
