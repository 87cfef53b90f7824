"""Brute force of the oracle against its scalar twin, decode validation classes,
and the plan's hand-computed decision table."""

import numpy as np
import pytest

from oracle import ciera_oracle as O
from oracle import naive as N


def test_every_change_mask_small_n():
    """All 2^n change masks for n <= 10 (B=64): numpy oracle == scalar twin,
    patches are exactly the masked positions, and decode restores x."""
    rng = np.random.default_rng(0)
    for n in range(1, 11):
        x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
        exact = O.exponent_field(x, O.BF16)
        for bits in range(1 << n):
            mask = np.array([(bits >> i) & 1 for i in range(n)], dtype=bool)
            cache = np.where(mask, exact ^ 0x40, exact).astype(np.uint8)
            s = O.encode(x, cache, O.BF16, 64, True)
            assert s.tobytes() == N.encode([int(v) for v in x], [int(v) for v in cache], 1, 64, True)
            h = O.parse_header(s)
            assert h["n_changed"] == mask.sum()
            out, c2, st = O.decode([s], n, 1, O.BF16, 64, 1, cache)
            assert st == 0 and np.array_equal(out, x) and np.array_equal(c2, exact)


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32, O.FP16])
def test_lengths_1_to_130_against_twin(dtype):
    """n in 1..130 with B=64 covers partial blocks and partial bitmap bytes."""
    rng = np.random.default_rng(dtype)
    bits = 32 if dtype == O.FP32 else 16
    for n in range(1, 131):
        x = rng.integers(0, 1 << bits, n, dtype=np.uint64).astype(O.int_dtype(dtype))
        exact = O.exponent_field(x, dtype)
        for f in (0.0, 0.05, 0.5):
            cache = np.where(rng.random(n) < f, exact ^ 0x81, exact).astype(np.uint8)
            for compress in (True, False):
                s = O.encode(x, cache, dtype, 64, compress, 3 * n, 3, 7)
                assert s.tobytes() == N.encode([int(v) for v in x], [int(v) for v in cache], dtype, 64,
                                               compress, 3 * n, 3, 7)
                vals, ex = N.decode(s.tobytes(), [int(v) for v in cache], dtype, 64)
                assert vals == [int(v) for v in x] and ex == [int(v) for v in exact]


# ------------------------------------------------------------- corruption

def _valid(n=3000, B=64, seed=1):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    exact = O.exponent_field(x, O.BF16)
    cache = np.where(rng.random(n) < 0.01, exact ^ 2, exact).astype(np.uint8)
    s = O.encode(x, cache, O.BF16, B, True)
    assert O.parse_header(s)["mode"] == O.MODE_COMPRESSED
    return x, cache, s


def _status(s, cache, n=3000, B=64, slot=None):
    slot_buf = np.zeros(slot if slot else max(s.size, 1), dtype=np.uint8)
    slot_buf[:s.size] = s[:slot_buf.size]
    return O.decode([slot_buf], n, 1, O.BF16, B, 1, cache)[2]


def _set(s, off, code_bytes):
    t = s.copy()
    t[off:off + len(code_bytes)] = np.frombuffer(code_bytes, dtype=np.uint8)
    return t


def test_corruption_classes():
    x, cache, s = _valid()
    n, B = 3000, 64
    p = O.parse_header(s)["n_changed"]
    nbm = O.bitmap_bytes(n, B)
    pb = 64 + n + nbm
    assert _status(s, cache) == 0
    assert _status(_set(s, 0, b"X"), cache) == O.ST_MAGIC
    assert _status(_set(s, 4, b"\x02\x00"), cache) == O.ST_MAGIC
    assert _status(_set(s, 6, b"\x02"), cache) == O.ST_FIELD            # dtype
    assert _status(_set(s, 7, b"\x05"), cache) == O.ST_FIELD            # mode
    assert _status(_set(s, 8, (128).to_bytes(4, "little")), cache) == O.ST_FIELD
    assert _status(_set(s, 16, (n - 1).to_bytes(8, "little")), cache) == O.ST_FIELD
    assert _status(_set(s, 40, (5).to_bytes(8, "little")), cache) == O.ST_FIELD
    assert _status(_set(s, 48, (1).to_bytes(4, "little")), cache) == O.ST_FIELD
    assert _status(_set(s, 52, (2).to_bytes(4, "little")), cache) == O.ST_FIELD
    assert _status(_set(s, 32, (s.size + 1).to_bytes(8, "little")), cache, slot=s.size + 8) == O.ST_LENGTH
    assert _status(_set(s, 24, (p + 1).to_bytes(8, "little")), cache, slot=s.size + 8) == O.ST_LENGTH
    assert _status(_set(s, 24, (n + 1).to_bytes(8, "little")), cache) == O.ST_LENGTH
    assert _status(s, cache, slot=s.size - 1) == O.ST_LENGTH           # truncated slot
    # patch index >= n
    assert _status(_set(s, pb + 5 * (p - 1), (n).to_bytes(4, "little")), cache) & O.ST_PATCH
    # two records swapped -> not ascending
    t = s.copy()
    t[pb:pb + 5], t[pb + 5:pb + 10] = s[pb + 5:pb + 10], s[pb:pb + 5]
    assert _status(t, cache) & O.ST_PATCH
    # duplicate record
    t = s.copy()
    t[pb + 5:pb + 10] = s[pb:pb + 5]
    assert _status(t, cache) & O.ST_PATCH
    # bitmap: clear a set bit / set a clear bit / set an unused tail bit
    bm = s[64 + n:64 + n + nbm]
    j = int(np.nonzero(bm)[0][0])
    bit = int(bm[j]) & -int(bm[j])
    assert _status(_set(s, 64 + n + j, bytes([bm[j] ^ bit])), cache) == O.ST_BITMAP
    zero_bits = np.nonzero(np.unpackbits(bm, bitorder="little")[:O.n_blocks(n, B)] == 0)[0]
    if zero_bits.size:
        b = int(zero_bits[0])
        assert _status(_set(s, 64 + n + b // 8, bytes([bm[b // 8] | (1 << (b % 8))])), cache) == O.ST_BITMAP
    nb = O.n_blocks(n, B)          # 47 blocks -> bit 47 of byte 5 is unused
    assert nb % 8 != 0
    assert _status(_set(s, 64 + n + nbm - 1, bytes([bm[-1] | 0x80])), cache) == O.ST_BITMAP


def test_status_is_format_validation_not_integrity():
    """Reading R36: the status bits flag streams that do not parse; edits that
    leave a well-formed stream decode with status 0 and a different output.
    Each case below is one such edit, with the exact status the oracle gives."""
    x, cache, s = _valid()
    n, B = 3000, 64
    p = O.parse_header(s)["n_changed"]
    pb = 64 + n + O.bitmap_bytes(n, B)
    recs = [(int.from_bytes(s[pb + 5 * k:pb + 5 * k + 4].tobytes(), "little"), int(s[pb + 5 * k + 4]))
            for k in range(p)]

    def dec(t):
        return O.decode([t], n, 1, O.BF16, B, 1, cache)

    out0 = dec(s)[0]
    assert np.array_equal(out0, x)
    # a sign|mantissa byte: not checked at all
    out, _, st = dec(_set(s, 64 + 17, bytes([s[64 + 17] ^ 0x01])))
    assert st == 0 and np.nonzero(out != x)[0].tolist() == [17]
    # a record's exponent byte: any value is a valid exponent
    out, _, st = dec(_set(s, pb + 4, bytes([s[pb + 4] ^ 0x01])))
    assert st == 0 and np.nonzero(out != x)[0].tolist() == [recs[0][0]]
    # a record's index moved inside its block, still between its neighbours:
    # the change lands on the wrong value (and the one it left keeps the cache)
    k = next(k for k in range(1, p - 1) if recs[k][0] % B != B - 1
             and recs[k][0] + 1 < recs[k + 1][0] and (recs[k][0] + 1) // B == recs[k][0] // B)
    i = recs[k][0]
    out, _, st = dec(_set(s, pb + 5 * k, (i + 1).to_bytes(4, "little")))
    assert st == 0 and set(np.nonzero(out != x)[0].tolist()) <= {i, i + 1} and not np.array_equal(out, x)
    # the same index moved into the next block: the bitmap no longer matches
    j = next(j for j in range(1, p - 1) if (recs[j - 1][0] // B) < (recs[j][0] // B) < (recs[j + 1][0] // B) - 1)
    to = (recs[j][0] // B + 1) * B
    assert _status(_set(s, pb + 5 * j, to.to_bytes(4, "little")), cache) == O.ST_BITMAP


# -------------------------------------------------------------------- plan
# Default cost model: link 8,000 B/us, HBM 5,600,000 B/us, fixed 5,000 ns,
# encode overlapped.  Worked by hand, W = 16, bf16, B = 512:
#
# RMSNorm 7168 (1-D, cols=1): n = 448, raw = 64 + 896 = 960.
#   P^ = ceil(10000*448/1e6) = ceil(4.48) = 5; nbm = ceil(ceil(448/512)/8) = 1
#   comp = 64 + 448 + 1 + 25 = 538
#   save = 422*15*1000 // 8000 = 791
#   dec  = 5000 + 16*(538 + 448 + 448 + 896)*1000 // 5600000 = 5000 + 6 = 5006
#   gain = -4215 -> RAW
# Router 7168x256: n = 448*256 = 114688, raw = 64 + 229376 = 229440.
#   P^ = ceil(1146.88) = 1147; nbm = ceil(224/8) = 28; comp = 64 + 114688 + 28 + 5735 = 120515
#   save = 108925*15000 // 8000 = 204234
#   dec  = 5000 + 16*579267*1000 // 5600000 = 5000 + 1655 = 6655
#   gain = 197579 -> COMPRESS
# OLMoE gate 2048x1024 fp32 at 30%: n = 131072, raw = 64 + 524288 = 524352.
#   P^ = 39322; comp = 64 + 393216 + 32 + 196610 = 589922 >= raw -> RAW, gain 0
# OLMoE gate 2048x1024 bf16 at 1%: n = 131072, raw = 262208.
#   P^ = ceil(1310.72) = 1311; comp = 64 + 131072 + 32 + 6555 = 137723
#   save = 124485*15000 // 8000 = 233409
#   dec  = 5000 + 16*(137723 + 262144 + 262144)*1000 // 5600000 = 5000 + 1891 = 6891
#   gain = 226518 -> COMPRESS
# Same tensor, W = 1: save = 0 -> gain = -dec -> RAW.
# OLMoE gate 2048x1024 fp16 at 1%: n = 131072, raw = 262208, sign|mantissa
#   ceil(11*131072/8) = 180224; comp = 64 + 180224 + 32 + 6555 = 186875
#   save = 75333*15000 // 8000 = 141249
#   dec  = 5000 + 16*(186875 + 262144 + 262144)*1000 // 5600000 = 5000 + 2031 = 7031
#   gain = 134218 -> COMPRESS
# RMSNorm 7168 fp16 at 1%: n = 448, raw = 960, sign|mantissa ceil(4928/8) = 616
#   comp = 64 + 616 + 1 + 25 = 706; save = 254*15000 // 8000 = 476
#   dec  = 5000 + 16*(706 + 448 + 448 + 896)*1000 // 5600000 = 5000 + 7 = 5007
#   gain = -4531 -> RAW
PLAN_TABLE = [
    # rows, cols, dtype, world, ppm, compress, expected bytes, gain
    (7168, 1, O.BF16, 16, 10000, 0, 960, -4215),
    (7168, 256, O.BF16, 16, 10000, 1, 120515, 197579),
    (2048, 1024, O.FP32, 16, 300000, 0, 524352, 0),
    (2048, 1024, O.BF16, 16, 10000, 1, 137723, 226518),
    (2048, 1024, O.FP16, 16, 10000, 1, 186875, 134218),
    (7168, 1, O.FP16, 16, 10000, 0, 960, -4531),
]


@pytest.mark.parametrize("row", PLAN_TABLE)
def test_plan_decision_table(row):
    rows, cols, dtype, world, ppm, compress, expected, gain = row
    p = O.plan(rows, cols, dtype, 512, world, ppm)
    assert p["compress"] == compress
    assert p["expected_stream_bytes"] == expected
    assert p["gain_ns"] == gain


def test_plan_edges():
    # no communication to save at W = 1 (the pages' Scout case: nothing selected -> baseline)
    assert O.plan(2048, 1024, O.BF16, 512, 1, 10000)["compress"] == 0
    # nothing changes -> payload is S_{s+m}: compress any large tensor
    p = O.plan(2048, 1024, O.BF16, 512, 16, 0)
    assert p["compress"] == 1 and p["expected_stream_bytes"] == 64 + 131072
    # byte break-even near 20% for both dtypes (5 bytes per patch vs 1 byte saved per value)
    assert O.plan(2048, 1024, O.BF16, 512, 16, 190000)["compress"] == 1
    assert O.plan(2048, 1024, O.BF16, 512, 16, 200000)["compress"] == 0
    assert O.plan(2048, 1024, O.FP32, 512, 16, 190000)["compress"] == 1
    assert O.plan(2048, 1024, O.FP32, 512, 16, 200000)["compress"] == 0
    # a non-overlapped encode adds its cost
    a = O.plan(2048, 1024, O.BF16, 512, 16, 10000)
    b = O.plan(2048, 1024, O.BF16, 512, 16, 10000, dict(overlap_encode=0))
    assert b["gain_ns"] < a["gain_ns"]
