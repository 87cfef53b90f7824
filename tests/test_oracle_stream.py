"""Pins of the oracle's stream format: hand-derived known-answer streams,
closed forms the pages fix, exhaustive round trips and the pages' block model.

The known-answer streams below were worked out by hand from the written format
(64-byte little-endian header; sign|mantissa bytes; bitmap LSB-first; 5-byte
(u32 index, u8 exponent) records) -- they do not come from running any code.
"""
import math

import numpy as np
import pytest

from oracle import ciera_oracle as O
from oracle import naive as N


def H(s: str) -> np.ndarray:
    return np.frombuffer(bytes.fromhex("".join(s.split())), dtype=np.uint8)


# --------------------------------------------------------- known answers

def kat_bf16():
    """n=130 bf16 values, B=64, rank 1 of 2 at element offset 130.
    All values are 1.0 (0x3F80: exponent 127, sign|mantissa 0x00) except
      x[0]   = -1.5 (0xBFC0) -> sign|mantissa 0xC0, exponent 127 (unchanged)
      x[3]   =  2.0 (0x4000) -> exponent 128, cache 127 -> patch (3, 0x80)
      x[64]  = -0.0 (0x8000) -> sign|mantissa 0x80, exponent 0 = cache
      x[129] =  0.5 (0x3F00) -> exponent 126, cache 127 -> patch (129, 0x7E)
    Blocks of 64: index 3 is in block 0 and index 129 in block 2 -> bitmap 0b101.
    total = 64 + 130 + 1 + 2*5 = 205 (0xCD) < raw 64 + 260."""
    x = np.full(130, 0x3F80, dtype=np.uint16)
    x[0], x[3], x[64], x[129] = 0xBFC0, 0x4000, 0x8000, 0x3F00
    cache = np.full(130, 127, dtype=np.uint8)
    cache[64] = 0
    smb = np.zeros(130, dtype=np.uint8)
    smb[0], smb[64] = 0xC0, 0x80
    want = np.concatenate([
        H("43494552 0100 01 01 40000000 00000000"
          "8200000000000000 0200000000000000 CD00000000000000 8200000000000000"
          "01000000 02000000 0000000000000000"),
        smb,
        H("05"),
        H("0300000080 810000007E"),
    ])
    return x, cache, want


def kat_fp32():
    """n=8 fp32 values, B=64, rank 0 of 1.  Only x[1] = -3.0 changes exponent
    (128 vs cached 127).  Sign|mantissa as 3 little-endian bytes each:
      1.0 -> 000000; -3.0 -> C00000; 1.5 -> 400000; smallest subnormal -> 000001;
      +Inf -> 000000; NaN 0xFFC00001 -> C00001; -0.0 -> 800000; 1.0 -> 000000.
    total = 64 + 24 + 1 + 5 = 94 (0x5E) < raw 96."""
    x = np.array([0x3F800000, 0xC0400000, 0x3FC00000, 0x00000001,
                  0x7F800000, 0xFFC00001, 0x80000000, 0x3F800000], dtype=np.uint32)
    cache = np.array([127, 127, 127, 0, 255, 255, 0, 127], dtype=np.uint8)
    want = H("43494552 0100 02 01 40000000 00000000"
             "0800000000000000 0100000000000000 5E00000000000000 0000000000000000"
             "00000000 01000000 0000000000000000"
             "000000 0000C0 000040 010000 000000 0100C0 000080 000000"
             "01"
             "0100000080")
    return x, cache, want


def kat_fp16():
    """n=16 fp16 values, B=64, rank 0 of 1.  11-bit sign|mantissa values
    (sign << 10 | mantissa) packed back to back, least significant bit first:
      x[0] =  1.0    0x3C00 -> sm 0x000, exponent 15
      x[1] = -2.0    0xC000 -> sm 0x400, exponent 16, cache 15 -> patch (1, 0x10)
      x[2] =  1.5    0x3E00 -> sm 0x200
      x[3] =  2^-24  0x0001 -> sm 0x001, exponent 0
      x[4] = +Inf    0x7C00 -> sm 0x000, exponent 31
      x[5] =  NaN    0xFE01 -> sm 0x601, exponent 31
      x[6] = -0.0    0x8000 -> sm 0x400, exponent 0
      x[7] = 65504   0x7BFF -> sm 0x3FF, exponent 30
      x[8..15] = 1.0 -> sm 0x000
    Set bits of the stream: 21 (x1), 31 (x2), 33 (x3), 55, 64, 65 (x5), 76 (x6),
    77..86 (x7) -> bytes 00 00 20 80 02 00 80 00 03 F0 7F, then 11 zero bytes
    (176 bits = 22 bytes).  total = 64 + 22 + 1 + 5 = 92 (0x5C) < raw 96."""
    x = np.array([0x3C00, 0xC000, 0x3E00, 0x0001, 0x7C00, 0xFE01, 0x8000, 0x7BFF] + [0x3C00] * 8,
                 dtype=np.uint16)
    cache = np.array([15, 15, 15, 0, 31, 31, 0, 30] + [15] * 8, dtype=np.uint8)
    want = H("43494552 0100 03 01 40000000 00000000"
             "1000000000000000 0100000000000000 5C00000000000000 0000000000000000"
             "00000000 01000000 0000000000000000"
             "0000208002008000 03F07F" + "00" * 11 +
             "01"
             "0100000010")
    return x, cache, want


def test_known_answer_fp16():
    x, cache, want = kat_fp16()
    got = O.encode(x, cache, O.FP16, 64, True)
    assert got.tobytes().hex() == want.tobytes().hex()
    assert N.encode([int(v) for v in x], [int(v) for v in cache], 3, 64, True) == want.tobytes()
    out, new_cache, st = O.decode([want], 16, 1, O.FP16, 64, 1, cache)
    assert st == 0 and np.array_equal(out, x) and new_cache[1] == 16


def test_known_answer_fp16_partial_group():
    """n=3 (33 bits -> 5 bytes), nothing changed, B=512:
      -0.0 (sm 0x400) -> bit 10; 65504 (sm 0x3FF) -> bits 11..20;
      NaN 0xFE01 (sm 0x601) -> bits 22, 31, 32  => 00 FC 5F 80 01.
    total = 64 + 5 = 69 (0x45) < raw 70."""
    x = np.array([0x8000, 0x7BFF, 0xFE01], dtype=np.uint16)
    cache = np.array([0, 30, 31], dtype=np.uint8)
    want = H("43494552 0100 03 01 00020000 00000000"
             "0300000000000000 0000000000000000 4500000000000000 0000000000000000"
             "00000000 01000000 0000000000000000"
             "00FC5F8001")
    assert O.encode(x, cache, O.FP16, 512, True).tobytes().hex() == want.tobytes().hex()
    assert N.encode([int(v) for v in x], [int(v) for v in cache], 3, 512, True) == want.tobytes()


def test_known_answer_bf16():
    x, cache, want = kat_bf16()
    got = O.encode(x, cache, O.BF16, 64, True, offset=130, rank=1, world=2)
    assert got.tobytes().hex() == want.tobytes().hex()
    assert N.encode([int(v) for v in x], [int(v) for v in cache], 1, 64, True, 130, 1, 2) == want.tobytes()


def test_known_answer_fp32():
    x, cache, want = kat_fp32()
    got = O.encode(x, cache, O.FP32, 64, True)
    assert got.tobytes().hex() == want.tobytes().hex()
    assert N.encode([int(v) for v in x], [int(v) for v in cache], 2, 64, True) == want.tobytes()


def test_known_answer_fp32_raw_fallback():
    """With only the first four fp32 values, 64 + 12 + 1 + 5 = 82 >= 80 = raw, so
    the stream is RAW: header (mode 0, n_changed 1, total 80) then the values."""
    x, cache, _ = kat_fp32()
    want = H("43494552 0100 02 00 40000000 00000000"
             "0400000000000000 0100000000000000 5000000000000000 0000000000000000"
             "00000000 01000000 0000000000000000"
             "0000803F 000040C0 0000C03F 01000000")
    got = O.encode(x[:4], cache[:4], O.FP32, 64, True)
    assert got.tobytes().hex() == want.tobytes().hex()


def test_known_answer_zero_change_and_plan_raw():
    """Nothing changed: header + exactly n sign|mantissa bytes, no bitmap."""
    x = np.full(20, 0xBF80, dtype=np.uint16)                 # -1.0: sign|mantissa 0x80
    cache = np.full(20, 127, dtype=np.uint8)
    want = np.concatenate([
        H("43494552 0100 01 01 00020000 00000000"
          "1400000000000000 0000000000000000 5400000000000000 0000000000000000"
          "00000000 01000000 0000000000000000"),
        np.full(20, 0x80, dtype=np.uint8)])
    assert O.encode(x, cache, O.BF16, 512, True).tobytes() == want.tobytes()
    # the plan said RAW: mode 0, the values little-endian, total 64 + 40 = 0x68
    raw = O.encode(x, cache, O.BF16, 512, False)
    assert raw[7] == 0 and raw[32] == 0x68 and raw.size == 104
    assert raw[64:].tobytes() == bytes.fromhex("80BF" * 20)


# ---------------------------------------------------- closed forms / invariants

@pytest.mark.parametrize("dtype", [O.BF16, O.FP32, O.FP16])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 511, 512, 513, 4096, 10000])
def test_zero_change_length(dtype, n):
    """No exponent changed -> exactly the sign|mantissa section plus the header:
    n bytes (bf16), 3n (fp32), ceil(11n/8) (fp16) -- RAW only on a tie with the
    raw length (one fp16 value: 2 bytes either way)."""
    rng = np.random.default_rng(n)
    x = rng.integers(0, 1 << (32 if dtype == O.FP32 else 16), n, dtype=np.uint64).astype(O.int_dtype(dtype))
    s = O.encode(x, O.exponent_field(x, dtype), dtype, 512, True)
    want = 64 + {O.BF16: n, O.FP32: 3 * n, O.FP16: (11 * n + 7) // 8}[dtype]
    raw = 64 + {O.BF16: 2, O.FP32: 4, O.FP16: 2}[dtype] * n
    if want < raw:
        assert s.size == want and O.parse_header(s)["mode"] == O.MODE_COMPRESSED
    else:
        assert dtype == O.FP16 and n == 1 and s.size == raw and O.parse_header(s)["mode"] == O.MODE_RAW


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32, O.FP16])
def test_all_changed_is_raw(dtype):
    """Every exponent differs: 5 bytes per patch exceed the (e-k) bytes saved -> RAW."""
    rng = np.random.default_rng(5)
    n = 1000
    x = rng.integers(0, 1 << (32 if dtype == O.FP32 else 16), n, dtype=np.uint64).astype(O.int_dtype(dtype))
    cache = O.exponent_field(x, dtype) ^ np.uint8(1)
    s = O.encode(x, cache, dtype, 512, True)
    h = O.parse_header(s)
    assert h["mode"] == O.MODE_RAW and h["n_changed"] == n and s.size == 64 + n * O.elem_bytes(dtype)


def test_tie_is_raw():
    """comp_len == raw_len -> RAW (R8).  bf16, B=512: 64+n+1+5P == 64+2n at n=11, P=2."""
    n, p = 11, 2
    assert O.comp_len(n, p, O.BF16, 512) == O.raw_len(n, O.BF16)
    x = np.full(n, 0x3F80, dtype=np.uint16)
    cache = np.full(n, 127, dtype=np.uint8)
    cache[[2, 7]] = 1
    assert O.parse_header(O.encode(x, cache, O.BF16, 512, True))["mode"] == O.MODE_RAW
    cache[7] = 127                                         # P=1 -> strictly shorter
    assert O.parse_header(O.encode(x, cache, O.BF16, 512, True))["mode"] == O.MODE_COMPRESSED


def test_payload_model_matches_pages():
    """[CIERA 3.2] expected payload S_{s+m} + S_bm + q*S_e with S_b = ceil(N/B),
    S_bm = ceil(S_b/8).  With q = 0 the payload is S_{s+m} only (bitmap omitted, R3);
    the changed exponents themselves cost one byte each plus a 4-byte index (R2)."""
    n, B = 131072 // 16, 512
    sb = math.ceil(n / B)
    sbm = math.ceil(sb / 8)
    s_sm = n * 1                       # bf16: 16 bits per value, 8 of them exponent
    assert O.bitmap_bytes(n, B) == sbm == 2
    assert O.comp_len(n, 0, O.BF16, B) - 64 == s_sm
    assert O.comp_len(n, 82, O.BF16, B) - 64 == s_sm + sbm + 82 * (1 + 4)


def test_exhaustive_bf16_round_trip():
    """decode(encode(x)) == x for all 65,536 bf16 patterns (+-0, subnormals, Inf,
    every NaN payload), against several caches, in one shard and sharded."""
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(7)
    exact = O.exponent_field(x, O.BF16)
    for cache in (exact, rng.integers(0, 256, x.size, dtype=np.uint8),
                  np.where(rng.random(x.size) < 0.01, exact ^ 1, exact).astype(np.uint8)):
        for world in (1, 4):
            rows, cols = 256, 256
            streams = [O.encode(x[o:o + n], cache[o:o + n], O.BF16, 512, True, o, r, world)
                       for r in range(world) for (o, n) in [O.shard(rows, cols, world, r)]]
            out, new_cache, st = O.decode(streams, rows, cols, O.BF16, 512, world, cache)
            assert st == 0
            assert np.array_equal(out, x)
            assert np.array_equal(new_cache, exact)          # cache == EXP(x) after decode


def test_exhaustive_fp16_round_trip():
    """decode(encode(x)) == x for all 65,536 fp16 patterns against several
    caches, in one shard and in shards whose lengths are not multiples of 8."""
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(8)
    exact = O.exponent_field(x, O.FP16)
    for cache in (exact, rng.integers(0, 32, x.size, dtype=np.uint8),
                  np.where(rng.random(x.size) < 0.01, exact ^ 1, exact).astype(np.uint8)):
        for rows, cols, world in ((256, 256, 1), (4096, 16, 4), (65536, 1, 7)):
            streams = [O.encode(x[o:o + n], cache[o:o + n], O.FP16, 512, True, o, r, world)
                       for r in range(world) for (o, n) in [O.shard(rows, cols, world, r)]]
            out, new_cache, st = O.decode(streams, rows, cols, O.FP16, 512, world, cache)
            assert st == 0 and np.array_equal(out, x) and np.array_equal(new_cache, exact)


def test_fp16_lengths_closed_form():
    """fp16 sign|mantissa section: 11 bits per value, ceil(11n/8) bytes; 8 values
    fill exactly 11 bytes; with no change the stream is 64 + ceil(11n/8)."""
    for n in range(0, 100):
        assert O.sm_section_bytes(n, O.FP16) == math.ceil(11 * n / 8)
        assert O.comp_len(n, 0, O.FP16, 64) == 64 + math.ceil(11 * n / 8)
    assert O.comp_len(8000, 0, O.FP16, 64) == 64 + 11000
    # ratio at no change: raw 2 bytes per value vs 11/8
    n = 1 << 20
    assert O.raw_len(n, O.FP16) - 64 == 2 * n and O.comp_len(n, 0, O.FP16, 512) - 64 == n * 11 // 8


def test_fp32_round_trip_structured():
    rng = np.random.default_rng(11)
    from tests.test_oracle_fields import fp32_structured
    x = np.concatenate([fp32_structured(), rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)])
    exact = O.exponent_field(x, O.FP32)
    cache = np.where(rng.random(x.size) < 0.02, exact ^ 3, exact).astype(np.uint8)
    s = O.encode(x, cache, O.FP32, 256, True)
    assert O.parse_header(s)["mode"] == O.MODE_COMPRESSED
    out, c2, st = O.decode([s], x.size, 1, O.FP32, 256, 1, cache)
    assert st == 0 and np.array_equal(out, x) and np.array_equal(c2, exact)


def test_bitmap_and_patch_invariants():
    rng = np.random.default_rng(3)
    for n, B, f in [(100_000, 512, 0.001), (100_000, 64, 0.01), (77_777, 4096, 0.05), (5000, 128, 0.0)]:
        x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
        exact = O.exponent_field(x, O.BF16)
        chg = rng.random(n) < f
        cache = np.where(chg, exact ^ 0x10, exact).astype(np.uint8)
        s = O.encode(x, cache, O.BF16, B, True)
        h = O.parse_header(s)
        p = h["n_changed"]
        assert p == chg.sum()
        if p == 0:
            assert s.size == 64 + n
            continue
        nbm = O.bitmap_bytes(n, B)
        bm = s[64 + n:64 + n + nbm]
        rec = s[64 + n + nbm:].reshape(p, 5)
        idx = rec[:, :4].copy().view("<u4").reshape(-1)
        assert np.all(np.diff(idx.astype(np.int64)) > 0) and idx.max() < n
        assert np.array_equal(idx, np.nonzero(chg)[0])
        assert np.array_equal(rec[:, 4], exact[idx])
        bits = np.unpackbits(bm, bitorder="little")
        assert bits.sum() == np.unique(idx // B).size
        assert np.all(bits[np.unique(idx // B)] == 1)


@pytest.mark.parametrize("f,B", [(0.001, 512), (0.01, 512), (0.003, 64), (0.1, 512)])
def test_block_change_density_matches_pages_model(f, B):
    """[CIERA 2.3] under a uniform per-element change rate c, a block of B values
    stays reusable with probability (1-c)^B.  The fraction of set bitmap bits must
    match 1-(1-f)^B within a 5-sigma binomial interval."""
    rng = np.random.default_rng(int(f * 1e6) + B)
    n = 4_000_000
    x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    exact = O.exponent_field(x, O.BF16)
    cache = np.where(rng.random(n) < f, exact ^ 1, exact).astype(np.uint8)
    s = O.encode(x, cache, O.BF16, B, True)
    nb = O.n_blocks(n, B)
    nbm = O.bitmap_bytes(n, B)
    bits = np.unpackbits(s[64 + n:64 + n + nbm], bitorder="little")[:nb]
    p = 1 - (1 - f) ** B
    sd = math.sqrt(p * (1 - p) / nb) + 1e-12
    assert abs(bits.mean() - p) <= 5 * sd + 1e-9, (bits.mean(), p)


def test_multi_iteration_cache_carry():
    """Iterates W0 -> W1 -> W2 -> W3 with 30%, 5%, 0.5% changes: every decode
    reproduces W_t bitwise and leaves cache == EXP(W_t)."""
    rng = np.random.default_rng(21)
    rows, cols, world, B = 64, 1000, 4, 512
    w = rng.integers(0, 1 << 32, rows * cols, dtype=np.uint64).astype(np.uint32)
    cache = O.cache_update(w, O.FP32)
    for f in (0.30, 0.05, 0.005):
        chg = rng.random(w.size) < f
        w = np.where(chg, w ^ np.uint32(1 << 24), w) ^ rng.integers(0, 1 << 23, w.size, dtype=np.uint64).astype(np.uint32)
        streams = []
        for r in range(world):
            off, n = O.shard(rows, cols, world, r)
            pl = O.plan(rows, cols, O.FP32, B, world, int(f * 1e6))
            streams.append(O.encode(w[off:off + n], cache[off:off + n], O.FP32, B, bool(pl["compress"]), off, r, world))
        out, cache, st = O.decode(streams, rows, cols, O.FP32, B, world, cache)
        assert st == 0 and np.array_equal(out, w)
        assert np.array_equal(cache, O.exponent_field(w, O.FP32))
