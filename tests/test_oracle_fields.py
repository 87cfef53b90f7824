"""Pins of the oracle's field split/merge against IEEE-754 facts and library routines.

[CIERA 3.1] splits every value into exponent bits and sign-plus-mantissa bits.
Which bits those are is fixed by IEEE-754 binary32, binary16 and bfloat16 (the
top 16 bits of a binary32).  The pins below check the oracle against ``math.frexp`` /
``numpy.frexp`` and against float arithmetic rebuilding each value from its
fields -- neither of which shares the oracle's bit formulas.
"""
import math
import struct

import numpy as np
import pytest

from oracle import ciera_oracle as O

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def bf16_to_float(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(u) << 16))[0]


def test_bf16_split_join_exhaustive():
    ex = O.exponent_field(ALL_BF16, O.BF16)
    sm = O.sign_mantissa_field(ALL_BF16, O.BF16)
    assert ex.dtype == np.uint8 and sm.max() <= 0xFF
    back = O.join_fields(sm, ex, O.BF16)
    assert np.array_equal(back, ALL_BF16)
    # the pair (exponent, sign|mantissa) is a bijection of the 65,536 patterns
    assert np.unique(ex.astype(np.uint32) << 8 | sm).size == 65536


def test_bf16_exponent_matches_frexp_exhaustive():
    ex = O.exponent_field(ALL_BF16, O.BF16)
    for u in range(65536):
        v = bf16_to_float(u)
        if math.isnan(v) or math.isinf(v):
            assert ex[u] == 255, hex(u)
        elif v == 0.0 or abs(v) < 2.0 ** -126:          # zero or subnormal
            assert ex[u] == 0, hex(u)
        else:
            m, e = math.frexp(v)                           # v = m * 2**e, 0.5 <= |m| < 1
            assert ex[u] == e - 1 + 127, hex(u)


def test_bf16_sign_mantissa_rebuilds_value_exhaustive():
    ex = O.exponent_field(ALL_BF16, O.BF16).astype(int)
    sm = O.sign_mantissa_field(ALL_BF16, O.BF16).astype(int)
    for u in range(65536):
        v = bf16_to_float(u)
        s, m = sm[u] >> 7, sm[u] & 0x7F
        if math.isnan(v):
            assert ex[u] == 255 and m != 0
            continue
        if math.isinf(v):
            assert m == 0 and (v < 0) == bool(s)
            continue
        if ex[u] == 0:
            rebuilt = (m / 128.0) * 2.0 ** -126
        else:
            rebuilt = (1 + m / 128.0) * 2.0 ** (ex[u] - 127)
        rebuilt = -rebuilt if s else rebuilt
        assert rebuilt == v and math.copysign(1, rebuilt) == math.copysign(1, v), hex(u)


def test_fp16_split_join_exhaustive():
    ex = O.exponent_field(ALL_BF16, O.FP16)
    sm = O.sign_mantissa_field(ALL_BF16, O.FP16)
    assert ex.max() == 31 and sm.max() == 0x7FF
    assert np.array_equal(O.join_fields(sm, ex, O.FP16), ALL_BF16)
    assert np.unique(ex.astype(np.uint32) << 11 | sm).size == 65536
    # the 11-bit values survive the bit-stream packing, at every length mod 8
    for n in (65536, 65535, 65533, 9, 1):
        assert np.array_equal(O.unpack_sm(O.pack_sm(sm[:n], O.FP16), O.FP16, n), sm[:n])
        assert O.pack_sm(sm[:n], O.FP16).size == -(-11 * n // 8)


def test_fp16_fields_match_numpy_float16_exhaustive():
    """Exponent field against frexp of numpy's binary16 values; sign|mantissa
    rebuilds every finite value by float arithmetic."""
    v = ALL_BF16.view(np.float16).astype(np.float64)
    ex = O.exponent_field(ALL_BF16, O.FP16).astype(np.int64)
    sm = O.sign_mantissa_field(ALL_BF16, O.FP16).astype(np.int64)
    finite = np.isfinite(v)
    normal = finite & (np.abs(v) >= 2.0 ** -14)
    _, e = np.frexp(v[normal])
    assert np.array_equal(ex[normal], e - 1 + 15)
    assert np.all(ex[~finite] == 31) and np.all(ex[finite & ~normal] == 0)
    m = sm & 0x3FF
    mag = np.where(ex == 0, m / 1024.0 * 2.0 ** -14, (1 + m / 1024.0) * np.exp2(ex - 15.0))
    rebuilt = np.where(sm >> 10 == 1, -mag, mag)
    assert np.array_equal(rebuilt[finite], v[finite])
    assert np.array_equal(np.signbit(rebuilt[finite]), np.signbit(v[finite]))   # -0.0 included
    assert np.all((m[np.isnan(v)] != 0)) and np.all(m[np.isinf(v)] == 0)


def fp32_structured():
    """All 256 exponents x both signs x mantissa edges {0, 1, 0x400000, 0x7FFFFF}."""
    vals = []
    for s in (0, 1):
        for e in range(256):
            for m in (0, 1, 0x400000, 0x7FFFFF):
                vals.append((s << 31) | (e << 23) | m)
    return np.array(vals, dtype=np.uint32)


def test_fp32_split_join_structured_and_random():
    rng = np.random.default_rng(1234)
    u = np.concatenate([fp32_structured(),
                        rng.integers(0, 1 << 32, 4_000_000, dtype=np.uint64).astype(np.uint32)])
    ex = O.exponent_field(u, O.FP32)
    sm = O.sign_mantissa_field(u, O.FP32)
    assert sm.max() < (1 << 24)
    assert np.array_equal(O.join_fields(sm, ex, O.FP32), u)
    # sign|mantissa bytes survive the 3-byte packing
    assert np.array_equal(O.unpack_sm(O.pack_sm(sm, O.FP32), O.FP32), sm)


def test_fp32_exponent_matches_numpy_frexp():
    rng = np.random.default_rng(99)
    u = np.concatenate([fp32_structured(),
                        rng.integers(0, 1 << 32, 1_000_000, dtype=np.uint64).astype(np.uint32)])
    v = u.view(np.float32)
    ex = O.exponent_field(u, O.FP32).astype(np.int64)
    finite = np.isfinite(v)
    normal = finite & (np.abs(v) >= np.float32(2.0 ** -126))
    _, e = np.frexp(v[normal].astype(np.float64))
    assert np.array_equal(ex[normal], e - 1 + 127)
    assert np.all(ex[~finite] == 255)
    assert np.all(ex[finite & ~normal] == 0)
    # sign|mantissa rebuild through float arithmetic for normals
    sm = O.sign_mantissa_field(u[normal], O.FP32).astype(np.int64)
    mag = (1 + (sm & 0x7FFFFF) / 2.0 ** 23) * np.exp2(ex[normal] - 127.0)
    rebuilt = np.where(sm >> 23 == 1, -mag, mag)
    assert np.array_equal(rebuilt, v[normal].astype(np.float64))


def test_known_values():
    # 1.0 = 2**0 -> biased exponent 127; -2.0 -> 128 with sign set; 0.5 -> 126
    cases = {0x3F80: (127, 0x00), 0xC000: (128, 0x80), 0x3F00: (126, 0x00),
             0xBFC0: (127, 0xC0), 0x8000: (0, 0x80), 0x0001: (0, 0x01),
             0x7F80: (255, 0x00), 0xFFC1: (255, 0xC1)}
    for u, (e, s) in cases.items():
        assert O.exponent_field(np.array([u], np.uint16), O.BF16)[0] == e
        assert O.sign_mantissa_field(np.array([u], np.uint16), O.BF16)[0] == s


@pytest.mark.parametrize("rows,cols,world", [(256, 512, 4), (2048, 1024, 16), (7168, 1, 16),
                                              (10, 3, 4), (3, 5, 8), (0, 7, 2), (17, 1, 16)])
def test_shard_partition(rows, cols, world):
    """Shards tile the tensor in rank order; sizes differ by at most one row (R12)."""
    pos = 0
    sizes = []
    for r in range(world):
        off, n = O.shard(rows, cols, world, r)
        assert off == pos and n % max(cols, 1) == 0
        pos += n
        sizes.append(n // max(cols, 1))
    assert pos == rows * cols
    assert max(sizes) - min(sizes) <= 1 and sizes == sorted(sizes, reverse=True)
