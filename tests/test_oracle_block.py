"""Pins of the oracle's block-hash variant [CIERA 3.1; Appendix A, Algorithm 1],
CPU only: the pages' own change detection -- a 128-bit hash per block from
two SplitMix64 hashes, a bitmap of the blocks whose hash changed, their
exponents sent whole."""
import numpy as np
import pytest

from oracle import ciera_oracle as O

M64 = O.MASK64


def _unxorshift(y, k):
    x = y
    for _ in range(64 // k + 1):
        x = y ^ (x >> k)
    return x


def _mix64_inverse(y):
    i1 = pow(0xBF58476D1CE4E5B9, -1, 1 << 64)
    i2 = pow(0x94D049BB133111EB, -1, 1 << 64)
    y = _unxorshift(y, 31)
    y = (y * i2) & M64
    y = _unxorshift(y, 27)
    y = (y * i1) & M64
    return _unxorshift(y, 30)


def test_splitmix64_published_outputs():
    """SplitMix64 (the page's ref. 22) from state 0: state += GAMMA, output =
    mix64(state); its published first three outputs."""
    s, out = 0, []
    for _ in range(3):
        s = (s + O.GAMMA) & M64
        out.append(O.mix64(s))
    assert out == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_mix64_is_a_bijection():
    rng = np.random.default_rng(0)
    vals = [0, 1, M64, 1 << 63, O.GAMMA] + [int(v) for v in rng.integers(0, 2**63, 2000, dtype=np.int64)]
    vals += [v | (1 << 63) for v in vals[5:200]]
    for v in vals:
        assert _mix64_inverse(O.mix64(v)) == v


def test_block_hash_position_length_and_avalanche():
    rng = np.random.default_rng(1)
    b = bytes(rng.integers(0, 256, 512, dtype=np.uint8))
    h = O.block_hash64(b, O.HASH_SEEDS[0])
    # two different 8-byte words swapped: position matters
    sw = b[8:16] + b[0:8] + b[16:]
    assert b[0:8] != b[8:16] and O.block_hash64(sw, O.HASH_SEEDS[0]) != h
    # a trailing zero byte: length matters even though the padding is zeros
    assert O.block_hash64(b[:-1], O.HASH_SEEDS[0]) != O.block_hash64(b[:-1] + b"\0", O.HASH_SEEDS[0])
    # the two halves differ
    assert O.block_hash64(b, O.HASH_SEEDS[1]) != h
    # avalanche: one flipped input bit flips about half of the output bits
    flips = []
    for t in range(1500):
        bb = bytearray(rng.integers(0, 256, 64, dtype=np.uint8))
        h0 = O.block_hash64(bytes(bb), O.HASH_SEEDS[t % 2])
        bit = int(rng.integers(0, 512))
        bb[bit // 8] ^= 1 << (bit % 8)
        flips.append(bin(h0 ^ O.block_hash64(bytes(bb), O.HASH_SEEDS[t % 2])).count("1"))
    assert 31.0 < float(np.mean(flips)) < 33.0 and min(flips) > 8


@pytest.mark.parametrize("n,B", [(1, 64), (64, 64), (65, 64), (1000, 64), (4096, 512), (5000, 4096), (9, 128)])
def test_block_hashes_equal_the_scalar_definition(n, B):
    """block_hashes (all blocks at once) against block_hash64 block by block."""
    ex = np.random.default_rng(n).integers(0, 256, n).astype(np.uint8)
    h = O.block_hashes(ex, B)
    for k in range(O.n_blocks(n, B)):
        b = ex[k * B:(k + 1) * B].tobytes()
        assert int(h[k, 0]) == O.block_hash64(b, O.HASH_SEEDS[0])
        assert int(h[k, 1]) == O.block_hash64(b, O.HASH_SEEDS[1])


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32, O.FP16])
@pytest.mark.parametrize("B", [64, 512])
def test_changed_blocks_match_exact_compare(dtype, B):
    """The hash marks exactly the blocks whose exponents differ (what the
    exact per-value compare of the element variant sees)."""
    rng = np.random.default_rng(B + dtype)
    n = 7 * B + 13  # a partial last block
    dt = O.int_dtype(dtype)
    x0 = rng.integers(0, np.iinfo(dt).max, n, dtype=np.uint64).astype(dt)
    ebits = {O.BF16: 7, O.FP32: 23, O.FP16: 10}[dtype]
    for trial in range(30):
        x1 = x0.copy()
        # flip the lowest exponent bit of a few positions, and mantissa bits everywhere
        pos = rng.choice(n, int(rng.integers(0, 6)), replace=False)
        x1[pos] ^= dt(1 << ebits)
        x1 ^= (rng.integers(0, 1 << ebits, n, dtype=np.uint64)).astype(dt)
        h0 = O.hash_seed(x0, dtype, B)
        h1 = O.hash_seed(x1, dtype, B)
        by_hash = np.any(h0 != h1, axis=1)
        e0, e1 = O.exponent_field(x0, dtype), O.exponent_field(x1, dtype)
        exact = np.array([np.any(e0[k * B:(k + 1) * B] != e1[k * B:(k + 1) * B])
                          for k in range(O.n_blocks(n, B))])
        assert np.array_equal(by_hash, exact), trial


def test_known_answer_block_stream():
    """bf16, n = 200, B = 64: blocks 0..3, the last one 8 values.  Exponent
    changes at values 70 (block 1) and 195 (block 3), mantissas changed
    everywhere.  The stream is the 64-byte header (mode 2, n_changed 2, total
    64 + 200 + 1 + 2 * 64 = 393), the 200 sign|mantissa bytes, bitmap 0b00001010,
    the 64 exponent bytes of block 1, then the 8 of block 3 and 56 zero bytes."""
    rng = np.random.default_rng(7)
    x0 = (rng.integers(0, 128, 200).astype(np.uint16) | (np.uint16(120) << 7)
          | (rng.integers(0, 2, 200).astype(np.uint16) << 15)).astype(np.uint16)
    x1 = x0 ^ rng.integers(0, 128, 200).astype(np.uint16)       # mantissa bits only
    x1[70] = (x1[70] & 0x807F) | (121 << 7)
    x1[195] = (x1[195] & 0x807F) | (119 << 7)
    s, h1 = O.encode_block(x1, O.hash_seed(x0, O.BF16, 64), O.BF16, 64, True, offset=5, rank=3, world=9)
    ex1 = ((x1 >> 7) & 0xFF).astype(np.uint8)
    want = bytearray(b"CIER") + (1).to_bytes(2, "little") + bytes([1, 2]) + (64).to_bytes(4, "little")
    want += bytes(4) + (200).to_bytes(8, "little") + (2).to_bytes(8, "little") + (393).to_bytes(8, "little")
    want += (5).to_bytes(8, "little") + (3).to_bytes(4, "little") + (9).to_bytes(4, "little") + bytes(8)
    want += bytes(((((x1 >> 8) & 0x80) | (x1 & 0x7F)).astype(np.uint8)))
    want += bytes([0b00001010])
    want += bytes(ex1[64:128]) + bytes(ex1[192:200]) + bytes(56)
    assert s.tobytes() == bytes(want)
    assert np.array_equal(h1, O.hash_seed(x1, O.BF16, 64))


def test_block_lengths_closed_form():
    rng = np.random.default_rng(3)
    for dtype in (O.BF16, O.FP32, O.FP16):
        dt = O.int_dtype(dtype)
        x = rng.integers(0, np.iinfo(dt).max, 1000, dtype=np.uint64).astype(dt)
        h = O.hash_seed(x, dtype, 64)
        s, _ = O.encode_block(x, h, dtype, 64, True)
        assert s.size == 64 + O.sm_section_bytes(1000, dtype)          # nothing changed
        assert O.parse_header(s)["mode"] == O.MODE_BLOCK
        s, h2 = O.encode_block(x, np.zeros_like(h), dtype, 64, True)   # every block "changed"
        nb = O.n_blocks(1000, 64)
        c_len = 64 + O.sm_section_bytes(1000, dtype) + O.bitmap_bytes(1000, 64) + nb * 64
        assert O.block_comp_len(1000, nb, dtype, 64) == c_len
        mode = O.MODE_BLOCK if c_len < 64 + 1000 * O.elem_bytes(dtype) else O.MODE_RAW
        assert O.parse_header(s)["mode"] == mode and s.size == min(c_len, 64 + 1000 * O.elem_bytes(dtype))
        s, _ = O.encode_block(x, np.zeros_like(h), dtype, 64, False)   # plan says RAW
        assert O.parse_header(s)["mode"] == O.MODE_RAW


def test_block_round_trip_all_bf16_patterns():
    x1 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(4)
    x0 = x1.copy()
    x0[rng.choice(65536, 20, replace=False)] ^= np.uint16(1 << 7)
    for B in (64, 512):
        cache = O.cache_update(x0, O.BF16)
        s, h1 = O.encode_block(x1, O.hash_seed(x0, O.BF16, B), O.BF16, B, True)
        assert O.parse_header(s)["mode"] == O.MODE_BLOCK
        out, ex, st = O.decode_stream(s, O.BF16, B, 65536, 0, 0, 1, cache)
        assert st == 0 and np.array_equal(out, x1) and np.array_equal(ex, O.cache_update(x1, O.BF16))
        assert np.array_equal(h1, O.hash_seed(x1, O.BF16, B))


def test_block_decode_status_classes():
    rng = np.random.default_rng(5)
    n, B = 900, 64  # 15 blocks: bit 7 of the second bitmap byte lies past the last block
    x0 = rng.integers(0, 65536, n).astype(np.uint16)
    x1 = x0.copy()
    x1[[10, 400, 890]] ^= np.uint16(1 << 7)
    cache = O.cache_update(x0, O.BF16)
    s, _ = O.encode_block(x1, O.hash_seed(x0, O.BF16, B), O.BF16, B, True)
    nbm = O.bitmap_bytes(n, B)
    bm0 = 64 + n

    def st(edit):
        t = s.copy()
        edit(t)
        return O.decode_stream(t, O.BF16, B, n, 0, 0, 1, cache)[2]

    assert st(lambda t: None) == 0
    assert st(lambda t: t.__setitem__(bm0, t[bm0] ^ 0x02)) == O.ST_BITMAP     # set bits != n_changed
    assert st(lambda t: t.__setitem__(bm0 + nbm - 1, t[bm0 + nbm - 1] | 0x80)) == O.ST_BITMAP  # past the last block
    assert st(lambda t: t.__setitem__(slice(24, 32), np.frombuffer((17).to_bytes(8, "little"), np.uint8))) == O.ST_LENGTH
    assert st(lambda t: t.__setitem__(slice(32, 40), np.frombuffer((s.size + 1).to_bytes(8, "little"), np.uint8))) == O.ST_LENGTH
    assert st(lambda t: t.__setitem__(7, 9)) == O.ST_FIELD


def test_block_multi_iteration_carry():
    """30% -> 5% -> 0.5% of values changing, hash cache and exponent cache carried."""
    rng = np.random.default_rng(6)
    n, B = 5000, 64
    x = rng.integers(0, 65536, n).astype(np.uint16)
    hashes, cache = O.hash_seed(x, O.BF16, B), O.cache_update(x, O.BF16)
    for f in (0.3, 0.05, 0.005):
        y = x ^ rng.integers(0, 128, n).astype(np.uint16)
        y[rng.random(n) < f] ^= np.uint16(1 << 7)
        s, hashes = O.encode_block(y, hashes, O.BF16, B, True)
        out, cache, st = O.decode_stream(s, O.BF16, B, n, 0, 0, 1, cache)
        assert st == 0 and np.array_equal(out, y)
        x = y
