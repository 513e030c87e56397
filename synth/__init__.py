"""Seeded synthetic inputs shared by the tests, the benchmark and smoke().

This module only draws random numbers and packs them into the storage formats;
it holds none of the method's arithmetic (no dequantisation, no products, no
normalisation).  Both the HIP path and the fp64 oracle consume its output.

Every tensor is identified by ``(seed, name)``.  The name is hashed to a 32-bit
tensor id; each tensor is cut into fixed-size chunks and chunk ``c`` of tensor
``t`` is drawn from its own Philox-4x64 stream keyed by ``(seed, t << 32 | c)``.
Philox is counter-based (Salmon et al., "Parallel random numbers: as easy as
1, 2, 3", SC'11), so any chunk can be regenerated alone and chunks can be drawn
in parallel threads.

Storage formats packed here (the block layouts the GGUF-style weights use):
  * Q4_0 block, 18 bytes: little-endian binary16 scale d, then 16 bytes of
    4-bit codes (the code bytes are uniform, so every code is uniform 0..15).
  * Q8_0 block, 34 bytes: little-endian binary16 scale d, then 32 int8 codes.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ELEMS = 1 << 21          # elements per independent stream for dense tensors
CHUNK_BYTES = 1 << 22          # target bytes per stream for quantised matrices

Q4_0_BLOCK_BYTES = 18
Q8_0_BLOCK_BYTES = 34
BLOCK_ELEMS = 32

_MASK64 = (1 << 64) - 1


def tensor_id(name: str) -> int:
    return zlib.crc32(name.encode("utf-8")) & 0xFFFFFFFF


def _stream(seed: int, name: str, chunk: int) -> np.random.Generator:
    key = ((seed & _MASK64) << 64) | (tensor_id(name) << 32) | (chunk & 0xFFFFFFFF)
    return np.random.Generator(np.random.Philox(key=key))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _run_chunks(fn, n_chunks: int) -> None:
    if n_chunks <= 1:
        for c in range(n_chunks):
            fn(c)
        return
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(fn, range(n_chunks)))


# --------------------------------------------------------------------------- dense
def normal_f32(seed: int, name: str, shape) -> np.ndarray:
    """fp32 N(0, 1) values, chunked Philox streams."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)

    def one(c):
        lo = c * CHUNK_ELEMS
        hi = min(n, lo + CHUNK_ELEMS)
        out[lo:hi] = _stream(seed, name, c).standard_normal(hi - lo, dtype=np.float32)

    _run_chunks(one, (n + CHUNK_ELEMS - 1) // CHUNK_ELEMS)
    return out.reshape(shape)


def uniform_f32(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    """fp32 values uniform in [lo, hi) (drawn in fp64, rounded to fp32)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)

    def one(c):
        a = c * CHUNK_ELEMS
        b = min(n, a + CHUNK_ELEMS)
        u = _stream(seed, name, c).random(b - a)
        out[a:b] = (lo + (hi - lo) * u).astype(np.float32)

    _run_chunks(one, (n + CHUNK_ELEMS - 1) // CHUNK_ELEMS)
    return out.reshape(shape)


def tokens(seed: int, name: str, count: int, vocab: int) -> np.ndarray:
    """int32 token ids uniform in [0, vocab)."""
    return _stream(seed, name, 0).integers(0, vocab, size=count, dtype=np.int64).astype(np.int32)


# --------------------------------------------------------------------------- quantised
def _rows_per_chunk(row_bytes: int) -> int:
    return max(1, CHUNK_BYTES // row_bytes)


def _scales_f16(g: np.random.Generator, count: int, lo: float, hi: float) -> np.ndarray:
    u = g.random(count)
    return (lo + (hi - lo) * u).astype(np.float16)   # round-to-nearest-even binary16


def q4_0_matrix(seed: int, name: str, n_rows: int, k: int,
                d_lo: float = 0.005, d_hi: float = 0.02, rows=None) -> np.ndarray:
    """Q4_0 matrix, ``n_rows`` rows of ``k // 32`` 18-byte blocks, row-major.

    Scales are binary16 uniform in [d_lo, d_hi]; code bytes are uniform.
    ``rows=(r0, r1)`` regenerates only that row range (bit-identical to the
    same rows of the full matrix).
    """
    assert k % BLOCK_ELEMS == 0
    nb = k // BLOCK_ELEMS
    row_bytes = nb * Q4_0_BLOCK_BYTES
    rpc = _rows_per_chunk(row_bytes)
    r0, r1 = (0, n_rows) if rows is None else rows
    out = np.empty((r1 - r0, nb, Q4_0_BLOCK_BYTES), dtype=np.uint8)
    c0, c1 = r0 // rpc, (r1 + rpc - 1) // rpc

    def one(c):
        ca, cb = c * rpc, min(n_rows, (c + 1) * rpc)
        g = _stream(seed, name, c)
        d = _scales_f16(g, (cb - ca) * nb, d_lo, d_hi)
        nbytes = (cb - ca) * nb * 16
        raw = g.bit_generator.random_raw((nbytes + 7) // 8).view(np.uint8)[:nbytes]
        blk = np.empty((cb - ca, nb, Q4_0_BLOCK_BYTES), dtype=np.uint8)
        blk[:, :, 0:2] = d.view(np.uint8).reshape(cb - ca, nb, 2)
        blk[:, :, 2:] = raw.reshape(cb - ca, nb, 16)
        a, b = max(ca, r0), min(cb, r1)
        out[a - r0:b - r0] = blk[a - ca:b - ca]

    _run_chunks(lambda i: one(c0 + i), c1 - c0)
    return out.reshape(r1 - r0, row_bytes)


def q8_0_matrix(seed: int, name: str, n_rows: int, k: int,
                d_lo: float = 0.002, d_hi: float = 0.01, rows=None) -> np.ndarray:
    """Q8_0 matrix, ``n_rows`` rows of ``k // 32`` 34-byte blocks, row-major.

    Scales are binary16 uniform in [d_lo, d_hi]; codes are int8 uniform in
    [-127, 127].
    """
    assert k % BLOCK_ELEMS == 0
    nb = k // BLOCK_ELEMS
    row_bytes = nb * Q8_0_BLOCK_BYTES
    rpc = _rows_per_chunk(row_bytes)
    r0, r1 = (0, n_rows) if rows is None else rows
    out = np.empty((r1 - r0, nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    c0, c1 = r0 // rpc, (r1 + rpc - 1) // rpc

    def one(c):
        ca, cb = c * rpc, min(n_rows, (c + 1) * rpc)
        g = _stream(seed, name, c)
        d = _scales_f16(g, (cb - ca) * nb, d_lo, d_hi)
        q = g.integers(-127, 128, size=(cb - ca, nb, 32), dtype=np.int16).astype(np.int8)
        blk = np.empty((cb - ca, nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
        blk[:, :, 0:2] = d.view(np.uint8).reshape(cb - ca, nb, 2)
        blk[:, :, 2:] = q.view(np.uint8)
        a, b = max(ca, r0), min(cb, r1)
        out[a - r0:b - r0] = blk[a - ca:b - ca]

    _run_chunks(lambda i: one(c0 + i), c1 - c0)
    return out.reshape(r1 - r0, row_bytes)
