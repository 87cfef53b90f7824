"""Scalar twin of the oracle -- TEST INFRASTRUCTURE ONLY.

Pure-Python loops over one value at a time, no numpy, written independently of
``ciera_oracle`` so that brute-force tests on tiny shards can compare the two.
Same format and readings as ``ciera_oracle`` (CIERA arXiv 2609.04609v1,
section 3.1 and Appendix A, Algorithm 1).
"""
from __future__ import annotations

import struct
from typing import List, Tuple

BF16, FP32, FP16 = 1, 2, 3


def _sizes(dtype: int) -> Tuple[int, int, int, int]:
    """(mantissa bits, exponent bits, element bytes, sign|mantissa bits)."""
    return {BF16: (7, 8, 2, 8), FP32: (23, 8, 4, 24), FP16: (10, 5, 2, 11)}[dtype]


def split(u: int, dtype: int) -> Tuple[int, int]:
    """(exponent, sign|mantissa) of one bit pattern."""
    shift, ebits, e, _ = _sizes(dtype)
    sign = u >> (8 * e - 1)
    exp = (u >> shift) & ((1 << ebits) - 1)
    mant = u & ((1 << shift) - 1)
    return exp, (sign << shift) | mant


def merge(exp: int, sm: int, dtype: int) -> int:
    shift, _, e, _ = _sizes(dtype)
    sign = sm >> shift
    mant = sm & ((1 << shift) - 1)
    return (sign << (8 * e - 1)) | (exp << shift) | mant


def encode(x: List[int], cache: List[int], dtype: int, block: int, compress: bool,
           offset: int = 0, rank: int = 0, world: int = 1) -> bytes:
    shift, _, e, kbits = _sizes(dtype)
    n = len(x)
    acc, nacc = 0, 0           # sign|mantissa bit stream, least significant bit first
    changed = []
    for i, u in enumerate(x):
        exp, sm = split(u, dtype)
        acc |= sm << nacc
        nacc += kbits
        if exp != cache[i]:
            changed.append((i, exp))
    sm_bytes = acc.to_bytes((nacc + 7) // 8, "little")
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
    shift, _, e, kbits = _sizes(dtype)
    (_, _, _, mode, _, _, n, p, total, _, _, _, _) = struct.unpack_from("<4sHBBIIQQQQIIQ", stream, 0)
    sms = (n * kbits + 7) // 8
    body = stream[64:total]
    if mode == 0:
        xs = [struct.unpack_from("<H" if e == 2 else "<I", body, i * e)[0] for i in range(n)]
        return xs, [split(u, dtype)[0] for u in xs]
    exps = list(cache)
    if p:
        nbm = ((n + block - 1) // block + 7) // 8
        base = sms + nbm
        for j in range(p):
            i, v = struct.unpack_from("<IB", body, base + 5 * j)
            exps[i] = v
    acc = int.from_bytes(body[:sms], "little")
    xs = []
    for i in range(n):
        sm = (acc >> (i * kbits)) & ((1 << kbits) - 1)
        xs.append(merge(exps[i], sm, dtype))
    return xs, exps
