"""Pins of the oracle's entropy-coded patch mode (mode 3), CPU only.

[CIERA 3.1] the sender compresses the changed exponents with ANS and the
receiver decodes them before the merge.  The oracle codes each change (its gap
from the previous change and its exponent relative to the cached one) with
range ANS (Duda) over interleaved states (Giesen).  The pins below are fixed
by that definition and by arithmetic done by hand: a worked two-symbol example,
the exact bit count of uniform symbols, the entropy bound of table symbols,
per-state independence of the interleaving, the symbol content of a
hand-worked chunk, the geometric model of the gap buckets, and known-answer
stream layouts."""
import math
import struct

import numpy as np
import pytest

from oracle import ciera_oracle as O

M = 1 << O.RANS_SCALE


def test_rans_worked_example():
    """Two exponent classes in one state, worked by hand.  Encoding runs
    backwards from x = 65536.  Class 1 (start 2032, f 2032): 65536 = 32*2032 +
    512, so x = 32*4096 + 512 + 2032 = 133616.  Class 0 (start 0, f 2032):
    133616 = 65*2032 + 1536, so x = 65*4096 + 1536 = 267776.  No word is
    written (both states stay below f * 2^20)."""
    subs = [[(0, 0, 2032, 12)], [(0, 2032, 2032, 12)]]
    states, words = O.rans_encode(subs, 1)
    assert states == [267776] and words == []
    # decoding: 267776 & 4095 = 1536 -> class 0, x = 2032*65 + 1536 = 133616;
    # 133616 & 4095 = 2544 -> class 1, x = 2032*32 + 2544 - 2032 = 65536.
    x = 267776
    assert x & 4095 == 1536 and 2032 * (x >> 12) + 1536 == 133616
    x = 133616
    assert 2032 <= (x & 4095) < 4064 and 2032 * (x >> 12) + (x & 4095) - 2032 == O.RANS_LOW


def test_rans_uniform_symbols_exact_length():
    """A uniform k-bit symbol multiplies the state by exactly 2^k and a word
    divides it by exactly 2^16, so with x starting at 2^16 (17 bits) the final
    state has 17 + sum(k) - 16 * words bits."""
    rng = np.random.default_rng(0)
    for trial in range(50):
        ks = [int(k) for k in rng.integers(0, 17, int(rng.integers(1, 300)))]
        subs = [[(0, int(rng.integers(0, 1 << k)) if k else 0, 1, k)] for k in ks]
        states, words = O.rans_encode(subs, 1)
        assert O.RANS_LOW <= states[0] < 1 << 32
        assert states[0].bit_length() == 17 + sum(ks) - 16 * len(words), trial


def test_rans_table_symbols_entropy_bound():
    """Each table symbol scales the state by 2^12 / f up to a relative error
    below f / x <= 2^12 / 2^16, so the information held by the words and the
    final state is within 0.1 bit per symbol of sum(log2(2^12 / f))."""
    rng = np.random.default_rng(1)
    for c in (1, 40, 300, 1024):
        f = O.gap_bucket_freqs(c, 4096)
        cum = [sum(f[:i]) for i in range(len(f))]
        for trial in range(5):
            m = int(rng.integers(50, 2000))
            syms = rng.choice(len(f), m, p=np.array(f) / M)
            subs = [[(0, cum[s], f[s], 12)] for s in syms]
            states, words = O.rans_encode(subs, 1)
            info = 16 * len(words) + math.log2(states[0]) - 16
            ideal = sum(math.log2(M / f[s]) for s in syms)
            assert abs(info - ideal) <= 0.1 * m + 1e-9, (c, trial, info, ideal)
            assert abs(info - ideal) <= 0.002 * m + 1.0, (c, trial, info, ideal)  # typical states are large


def test_interleaved_states_match_single_state_coding():
    """States are independent: each state's final value equals coding its
    own symbols alone, and the words are the union of theirs."""
    rng = np.random.default_rng(2)
    for trial in range(40):
        length = int(rng.integers(1, 4097))
        c = int(rng.integers(1, min(length, 1024) + 1))
        offs = sorted(int(v) for v in rng.choice(length, c, replace=False))
        olds = [int(v) for v in rng.integers(0, 256, c)]
        news = [(o + int(rng.choice([1, 255, 3, 250, 128]))) & 0xFF for o in olds]
        subs, L = O._chunk_symbols(offs, olds, news, length)
        states, words = O.rans_encode(subs, L)
        assert L == O.rans_lanes(c)
        total = 0
        for lane in range(L):
            own = [[(0, s, f, k) for (l2, s, f, k) in sub if l2 == lane] for sub in subs]
            st1, w1 = O.rans_encode(own, 1)
            assert st1[0] == states[lane], (trial, lane)
            total += len(w1)
        assert total == len(words)


def test_lane_counts():
    assert [O.rans_lanes(c) for c in (1, 4, 5, 8, 9, 100, 252, 253, 256, 1024, 4096)] == \
        [1, 1, 2, 2, 3, 25, 63, 64, 64, 64, 64]


def test_chunk_symbols_worked_by_hand():
    """Changes at chunk offsets 0, 5, 6, 300 with exponent steps +1, -1, +9, -7
    (one state: c = 4).  Gaps 0, 4, 0, 293; buckets (bit length of gap + 1)
    1, 3, 1, 9; bits below the leading one: none, 5 - 4 = 1 (2 bits), none,
    294 - 256 = 38 (8 bits); classes 0 (+1), 1 (-1), 14 (escape: +9, the new
    exponent 109 sent as 8 bits), 13 (-7)."""
    length = 1000
    offs, olds = [0, 5, 6, 300], [120, 120, 100, 130]
    news = [121, 119, 109, 123]
    gf = O.gap_bucket_freqs(4, length)
    gc = [sum(gf[:i]) for i in range(13)]
    df = O.DELTA_FREQ
    dc = [sum(df[:i]) for i in range(15)]
    A = lambda b: [(0, gc[b - 1], gf[b - 1], 12)]
    C = lambda k: [(0, dc[k], df[k], 12)]
    want = [A(1), [], C(0), [],
            A(3), [(0, 1, 1, 2)], C(1), [],
            A(1), [], C(14), [(0, 109, 1, 8)],
            A(9), [(0, 38, 1, 8)], C(13), []]
    subs, L = O._chunk_symbols(offs, olds, news, length)
    assert L == 1 and subs == want


def test_delta_classes():
    assert sum(O.DELTA_FREQ) == M and len(O.DELTA_FREQ) == 15
    want = {1: 0, 255: 1, 2: 2, 254: 3, 3: 4, 253: 5, 7: 12, 249: 13}
    for d, cls in want.items():
        assert O.delta_class(100, (100 + d) & 0xFF) == cls
        assert O.class_delta(cls) == d
    for d in (8, 248, 128, 0):
        assert O.delta_class(100, (100 + d) & 0xFF) == O.DELTA_ESCAPE
    for old in range(256):                 # wraps modulo 256
        for cls in range(14):
            assert O.delta_class(old, (old + O.class_delta(cls)) & 0xFF) == cls


@pytest.mark.parametrize("c,length", [(1, 4096), (41, 4096), (410, 4096), (1024, 4096), (4096, 4096),
                                      (3, 100), (1, 1), (7, 9), (2000, 3000)])
def test_gap_buckets_follow_the_geometric_model(c, length):
    """Frequencies sum to 2^12, none is zero, and all but the largest lie
    within 1 of 2^12 times the geometric bucket probability (1-p)^(2^(b-1)-1)
    - (1-p)^(2^b - 1), the last bucket taking the tail; the largest absorbs
    the rounding (at most 13)."""
    f = O.gap_bucket_freqs(c, length)
    assert len(f) == 13 and sum(f) == M and min(f) >= 1
    q = 1.0 - c / length
    S = [q ** (2 ** i - 1) for i in range(13)]
    pr = [S[b - 1] - S[b] for b in range(1, 13)] + [S[12]]
    top = f.index(max(f))
    for b in range(13):
        tol = 14 if b == top else 1.01
        assert abs(f[b] - max(1.0, M * pr[b])) <= tol, (b, f[b], M * pr[b])


def test_gap_buckets_all_changed():
    """c = length: every gap is 0, so bucket 1 holds everything; the other
    twelve get the minimum 1 and bucket 1 gets 4096 - 12."""
    assert O.gap_bucket_freqs(4096, 4096) == [4084] + [1] * 12
    assert O.gap_bucket_freqs(5, 5) == [4084] + [1] * 12


def _bf16_with_changes(n, changes, seed):
    """bf16 values whose exponents are 120 +- small, and a copy with the given
    exponent steps {index: step}."""
    rng = np.random.default_rng(seed)
    x0 = ((rng.integers(0, 2, n).astype(np.uint16) << 15) | (np.uint16(120) << 7)
          | rng.integers(0, 128, n).astype(np.uint16)).astype(np.uint16)
    x1 = x0 ^ rng.integers(0, 128, n).astype(np.uint16)          # mantissas change everywhere
    for i, d in changes.items():
        x1[i] = (x1[i] & 0x807F) | (((120 + d) & 0xFF) << 7)
    return x0, x1


def test_known_answer_stream_layout():
    """n = 8192 bf16, B = 64: chunk 0 has 1100 changes (more than 1024: sent
    dense, its 4096 exponent bytes), chunk 1 has 10 (rANS).  Stream: header
    (mode 3, n_changed 1110) | 8192 sign|mantissa bytes | 16 bitmap bytes
    (positions 8256..8271; 8272 is a multiple of 4, no padding) | table
    (1100, 4096), (1110, 4096 + D1) | dense chunk | rANS chunk."""
    rng = np.random.default_rng(3)
    ch = {int(i): 1 for i in rng.choice(4096, 1100, replace=False)}
    ch.update({4096 + int(i): -1 for i in rng.choice(4096, 10, replace=False)})
    x0, x1 = _bf16_with_changes(8192, ch, 4)
    cache = O.cache_update(x0, O.BF16)
    s = O.encode_coded(x1, cache, O.BF16, 64, True, offset=7, rank=1, world=2)
    ex1 = ((x1 >> 7) & 0xFF).astype(np.uint8)
    d1 = O.encode_chunk(ex1[4096:], cache[4096:])
    assert 8 <= len(d1) < 4096 and len(d1) % 4 == 0
    total = 8272 + 16 + 4096 + len(d1)
    want = bytearray(b"CIER") + (1).to_bytes(2, "little") + bytes([1, 3]) + (64).to_bytes(4, "little")
    want += bytes(4) + (8192).to_bytes(8, "little") + (1110).to_bytes(8, "little") + total.to_bytes(8, "little")
    want += (7).to_bytes(8, "little") + (1).to_bytes(4, "little") + (2).to_bytes(4, "little") + bytes(8)
    want += bytes(((((x1 >> 8) & 0x80) | (x1 & 0x7F)).astype(np.uint8)))
    bm = np.zeros(16, dtype=np.uint8)
    for i in ch:
        bm[(i // 64) // 8] |= 1 << ((i // 64) % 8)
    want += bytes(bm)
    want += struct.pack("<IIII", 1100, 4096, 1110, 4096 + len(d1))
    want += bytes(ex1[:4096]) + d1
    assert s.tobytes() == bytes(want)
    out, ex, st = O.decode_stream(s, O.BF16, 64, 8192, 7, 1, 2, cache, coded=True)
    assert st == 0 and np.array_equal(out, x1)


def test_known_answer_padding_and_no_change():
    """n = 100 bf16, B = 64: header, 100 sign|mantissa bytes, 1 bitmap byte at
    164, 3 zero bytes to 168, one table entry, the chunk data.  With no change
    the stream is header + sign|mantissa only, still mode 3."""
    x0, x1 = _bf16_with_changes(100, {3: 1, 70: -1, 71: 2}, 5)
    cache = O.cache_update(x0, O.BF16)
    s = O.encode_coded(x1, cache, O.BF16, 64, True)
    ex1 = ((x1 >> 7) & 0xFF).astype(np.uint8)
    d = O.encode_chunk(ex1, cache)
    assert len(d) == 4 + 4 * ((len(d) - 4) // 4) and len(d) < 100
    assert O.parse_header(s)["total_len"] == 168 + 8 + len(d) == s.size
    assert s[164] == 0b11 and s[165:168].tolist() == [0, 0, 0]
    assert struct.unpack_from("<II", s.tobytes(), 168) == (3, len(d))
    assert s[176:].tobytes() == d
    s0 = O.encode_coded(x0, cache, O.BF16, 64, True)
    assert O.parse_header(s0)["mode"] == O.MODE_CODED and s0.size == 164
    # a receiver that did not declare the tensor coded rejects mode 3 as a field mismatch
    assert O.decode_stream(s, O.BF16, 64, 100, 0, 0, 1, cache)[2] == O.ST_FIELD
    assert O.decode_stream(s, O.BF16, 64, 100, 0, 0, 1, cache, coded=True)[2] == 0
    assert O.parse_header(O.encode_coded(x1, cache, O.BF16, 64, False))["mode"] == O.MODE_RAW


def test_dense_threshold():
    """A chunk of 1024 changes is rANS data (much shorter than 4096 bytes at
    +-1 steps); 1025 changes make it dense."""
    rng = np.random.default_rng(6)
    old = rng.integers(100, 140, 4096).astype(np.uint8)
    for c, dense in ((1024, False), (1025, True)):
        new = old.copy()
        pos = rng.choice(4096, c, replace=False)
        new[pos] = (new[pos] + rng.choice([1, 255], c)).astype(np.uint8)
        d = O.encode_chunk(new, old)
        assert (d == new.tobytes()) == dense
        if not dense:
            assert len(d) < 1200


def test_round_trip_random_chunks_and_specials():
    rng = np.random.default_rng(7)
    for dt in (O.BF16, O.FP32, O.FP16):
        idt = O.int_dtype(dt)
        shift, em = {O.BF16: (7, 0xFF), O.FP32: (23, 0xFF), O.FP16: (10, 0x1F)}[dt]
        for n, f in ((1, 1.0), (4095, 0.01), (4097, 0.02), (12000, 0.1), (9000, 0.26), (3000, 0.5)):
            x0 = rng.integers(0, np.iinfo(idt).max, n, dtype=np.uint64).astype(idt)
            e0 = ((x0 >> shift) & em).astype(np.int64)
            m = rng.random(n) < f
            step = rng.choice([1, -1, 2, -7, 8, 100], n, p=[.4, .4, .05, .05, .05, .05])
            e1 = np.where(m, (e0 + step) % (em + 1), e0)
            x1 = ((x0 & ~idt(em << shift)) | (e1.astype(idt) << shift)).astype(idt)
            cache = O.cache_update(x0, dt)
            s = O.encode_coded(x1, cache, dt, 64, True, 0, 0, 1)
            out, ex, st = O.decode_stream(s, dt, 64, n, 0, 0, 1, cache, coded=True)
            assert st == 0 and np.array_equal(out, x1) and np.array_equal(ex, O.cache_update(x1, dt)), (dt, n, f)


def test_bits_per_change_near_entropy():
    """Size of the coded data at 1% uniform +-1 changes, bounded by bit
    accounting.  Information per change: the entropy of a geometric gap with
    p = 0.01, (-(1-p) log2(1-p) - p log2 p) / p = 8.08 bits, plus the class
    (+1 or -1, frequency 2032 of 4096 each): 1.01 bits.  Per state: encoding
    starts at 2^16 and every emitted word takes 16 bits out of the state, so a
    state that absorbed I bits and emitted w words ends at log2 x = 16 + I - 16w,
    and its stored bits are 32 + 16w = I + 48 - log2 x; a final state lies in
    [2^16, 2^32), so each state costs between 16 and 32 bits beyond its
    information.  Per chunk: at most one 16-bit padding word.  Hence
    9.09 + 16 L / c <= bits per change <= 9.09 + (32 L + 16 chunks) / c, L the
    states over all chunks; 0.5 bit of slack covers the table's rounding of
    the frequencies and the sample's deviation from the entropy.  Against 40
    bits as a (u32, u8) record."""
    rng = np.random.default_rng(8)
    n = 131072
    old = rng.integers(100, 130, n).astype(np.uint8)
    m = rng.random(n) < 0.01
    new = np.where(m, (old.astype(int) + rng.choice([1, -1], n)) % 256, old).astype(np.uint8)
    tot = lanes = 0
    for k in range(O.n_chunks(n)):
        a, b = new[k * 4096:(k + 1) * 4096], old[k * 4096:(k + 1) * 4096]
        tot += len(O.encode_chunk(a, b))
        lanes += -(-int(np.count_nonzero(a != b)) // 4)   # one state per 4 changes (<= 64 here)
    c = int(m.sum())
    bits = 8 * tot / c
    p = 0.01
    info = (-(1 - p) * math.log2(1 - p) - p * math.log2(p)) / p - math.log2(2032 / 4096)
    lo = info + 16 * lanes / c
    hi = info + (32 * lanes + 16 * O.n_chunks(n)) / c
    assert 13.0 < lo and hi < 18.0                      # the bound itself: 13.3 .. 17.8 bits
    assert lo - 0.5 < bits < hi + 0.5, (lo, bits, hi)


def _coded_case(n=12000, f=0.02, seed=9):
    rng = np.random.default_rng(seed)
    ch = {int(i): int(rng.choice([1, -1, 9])) for i in np.nonzero(rng.random(n) < f)[0]}
    x0, x1 = _bf16_with_changes(n, ch, seed)
    cache = O.cache_update(x0, O.BF16)
    return O.encode_coded(x1, cache, O.BF16, 64, True), cache, n


def _status(s, cache, n):
    return O.decode_stream(s, O.BF16, 64, n, 0, 0, 1, cache, coded=True)[2]


def test_coded_decode_status_classes():
    s, cache, n = _coded_case()
    assert O.parse_header(s)["mode"] == O.MODE_CODED and _status(s, cache, n) == 0
    tpos = O.pad4(64 + n + O.bitmap_bytes(n, 64))
    nch = O.n_chunks(n)
    dpos = tpos + 8 * nch
    tab = list(struct.unpack_from(f"<{2 * nch}I", s.tobytes(), tpos))

    def edit(pos, val):
        t = s.copy()
        t[pos:pos + 4] = np.frombuffer(struct.pack("<I", val), dtype=np.uint8)
        return _status(t, cache, n)

    assert edit(tpos + 8, tab[2] + 1) & O.ST_PATCH                   # one change moved between chunks
    assert edit(tpos + 8 * (nch - 1), tab[-2] + 1) & O.ST_LENGTH     # last count other than n_changed
    assert edit(tpos + 4, tab[1] + 4) & O.ST_PATCH                   # 4 bytes moved between chunks
    assert edit(tpos + 8 * (nch - 1) + 4, tab[-1] - 4) & O.ST_LENGTH  # last entry short of the data
    assert edit(tpos + 0, tab[2] + 1) & O.ST_LENGTH                  # goes backwards
    assert edit(tpos + 4, tab[1] + 2) & O.ST_LENGTH                  # not a multiple of 4
    # Flips inside chunk 0's first state (reading R36: status is format
    # validation, not an integrity check).  The bucket step passes the slot's
    # low bits through to the state and the raw-bits step of the same change
    # takes them out again, so a flip of the state's lowest bits changes only
    # the first gap: every change of the chunk moves by the same amount and the
    # rANS checks (words, final states) all pass.
    out0 = O.decode_stream(s, O.BF16, 64, n, 0, 0, 1, cache, coded=True)[0]
    t = s.copy()                                                      # bit 0: each change one place up;
    t[dpos] ^= 1                                                      # those at 639 and 1151 change block
    assert _status(t, cache, n) == O.ST_BITMAP
    t = s.copy()                                                      # bit 1: two places down, no block
    t[dpos] ^= 2                                                      # changes: not detected
    out, _, st = O.decode_stream(t, O.BF16, 64, n, 0, 0, 1, cache, coded=True)
    assert st == 0 and not np.array_equal(out, out0)
    t = s.copy()                                                      # bit 20, above the 12-bit slot: the
    t[dpos + 2] ^= 0x10                                               # buckets change, the words run out
    assert _status(t, cache, n) == O.ST_PATCH | O.ST_BITMAP
    t = s.copy()                                                      # total beyond the data
    t[32:40] = np.frombuffer((s.size + 4).to_bytes(8, "little"), dtype=np.uint8)
    assert _status(np.concatenate([t, np.zeros(4, np.uint8)]), cache, n) & O.ST_LENGTH
    t = s.copy()                                                      # total short of the table
    t[32:40] = np.frombuffer((dpos - 1).to_bytes(8, "little"), dtype=np.uint8)
    assert _status(t, cache, n) == O.ST_LENGTH


def test_coded_decode_flags_words_and_ranges():
    """Words missing, a change past its chunk, a dense chunk whose differences
    disagree with its count, an fp16 exponent wider than 5 bits."""
    rng = np.random.default_rng(10)
    old = rng.integers(10, 20, 4096).astype(np.uint8)
    new = old.copy()
    pos = rng.choice(4096, 300, replace=False)
    new[pos] = new[pos] + 1
    d = O.encode_chunk(new, old)
    L = O.rans_lanes(300)
    assert O.rans_decode_chunk(d, 300, 4096, old, 0xFF)[2] == 0
    assert O.rans_decode_chunk(d[:-4], 300, 4096, old, 0xFF)[2] & O.ST_PATCH       # words missing
    assert O.rans_decode_chunk(d + bytes(4), 300, 4096, old, 0xFF)[2] & O.ST_PATCH  # words left over
    assert O.rans_decode_chunk(d, 300, int(pos.max()), old, 0xFF)[2] & O.ST_PATCH  # a change past the chunk
    assert O.rans_decode_chunk(d, 300, 4096, old, 0x0F)[2] & O.ST_PATCH            # exponents too wide
    assert len(d) >= 4 * L
    # dense: one byte changed back to the cached value -> 1100 becomes 1099 differences
    x0, x1 = _bf16_with_changes(8192, {int(i): 1 for i in rng.choice(4096, 1100, replace=False)}, 11)
    cache = O.cache_update(x0, O.BF16)
    s = O.encode_coded(x1, cache, O.BF16, 64, True)
    dpos = 8272 + 16
    i = int(np.nonzero(((x1 >> 7) & 0xFF).astype(np.uint8)[:4096] != cache[:4096])[0][0])
    t = s.copy()
    t[dpos + i] = cache[i]
    assert O.decode_stream(t, O.BF16, 64, 8192, 0, 0, 1, cache, coded=True)[2] & O.ST_PATCH
