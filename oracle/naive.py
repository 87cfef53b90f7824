"""Scalar twin of the oracle -- TEST INFRASTRUCTURE ONLY.

Pure-Python loops over one value at a time, no numpy, written independently of
``ciera_oracle`` so that brute-force tests on tiny shards can compare the two.
Same format and readings as ``ciera_oracle`` (CIERA arXiv 2609.04609v1,
section 3.1 and Appendix A, Algorithm 1).
"""
from __future__ import annotations

import struct
from typing import List, Tuple

BF16, FP32 = 1, 2


def _sizes(dtype: int) -> Tuple[int, int, int]:
    """(exponent shift, element bytes, sign|mantissa bytes)."""
    return (7, 2, 1) if dtype == BF16 else (23, 4, 3)


def split(u: int, dtype: int) -> Tuple[int, int]:
    """(exponent, sign|mantissa) of one bit pattern."""
    shift, e, _ = _sizes(dtype)
    sign = u >> (8 * e - 1)
    exp = (u >> shift) & 0xFF
    mant = u & ((1 << shift) - 1)
    return exp, (sign << shift) | mant


def merge(exp: int, sm: int, dtype: int) -> int:
    shift, e, _ = _sizes(dtype)
    sign = sm >> shift
    mant = sm & ((1 << shift) - 1)
    return (sign << (8 * e - 1)) | (exp << shift) | mant


def encode(x: List[int], cache: List[int], dtype: int, block: int, compress: bool,
           offset: int = 0, rank: int = 0, world: int = 1) -> bytes:
    shift, e, k = _sizes(dtype)
    n = len(x)
    sm_bytes = bytearray()
    changed = []
    for i, u in enumerate(x):
        exp, sm = split(u, dtype)
        for b in range(k):
            sm_bytes.append((sm >> (8 * b)) & 0xFF)
        if exp != cache[i]:
            changed.append((i, exp))
    nblk = (n + block - 1) // block
    nbm = (nblk + 7) // 8
    bitmap = bytearray(nbm)
    for i, _ in changed:
        blk = i // block
        bitmap[blk // 8] |= 1 << (blk % 8)
    patches = bytearray()
    for i, exp in changed:
        patches += struct.pack("<IB", i, exp)
    body_c = bytes(sm_bytes) + (bytes(bitmap) + bytes(patches) if changed else b"")
    raw = b"".join(struct.pack("<H" if e == 2 else "<I", u) for u in x)
    use_c = compress and len(body_c) < len(raw)
    body = body_c if use_c else raw
    hdr = struct.pack("<4sHBBIIQQQQIIQ", b"CIER", 1, dtype, 1 if use_c else 0, block, 0,
                      n, len(changed), 64 + len(body), offset, rank, world, 0)
    return hdr + body


def decode(stream: bytes, cache: List[int], dtype: int, block: int) -> Tuple[List[int], List[int]]:
    """Decode one well-formed stream; returns (values, new cache)."""
    shift, e, k = _sizes(dtype)
    (_, _, _, mode, _, _, n, p, total, _, _, _, _) = struct.unpack_from("<4sHBBIIQQQQIIQ", stream, 0)
    body = stream[64:total]
    if mode == 0:
        xs = [struct.unpack_from("<H" if e == 2 else "<I", body, i * e)[0] for i in range(n)]
        return xs, [split(u, dtype)[0] for u in xs]
    exps = list(cache)
    if p:
        nbm = ((n + block - 1) // block + 7) // 8
        base = n * k + nbm
        for j in range(p):
            i, v = struct.unpack_from("<IB", body, base + 5 * j)
            exps[i] = v
    xs = []
    for i in range(n):
        sm = 0
        for b in range(k):
            sm |= body[i * k + b] << (8 * b)
        xs.append(merge(exps[i], sm, dtype))
    return xs, exps
