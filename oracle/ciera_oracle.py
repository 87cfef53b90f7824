"""CPU oracle of the CIERA exponent-reuse codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The product path (the HIP
library and its Python binding) never does, and shares no code with it.

It is plain, slow and written to be checked by eye against the pages:

  CIERA: Cross-Iteration Exponent Reuse for Lossless Allgather in Sharded MoE
  Training (arXiv 2609.04609v1), cited below as [CIERA].

  * [CIERA section 3.1] every value is split into its exponent bits and its
    sign-plus-mantissa bits; the exponents of the previous iteration are
    cached; the sender transmits the sign-plus-mantissa bits of every value,
    a bitmap with one bit per block of B values marking the blocks whose
    exponents changed, and the changed exponents; the receiver takes the old
    exponents from its cache, replaces the changed ones and merges them with
    the received sign-plus-mantissa bits.  Reconstruction is bitwise exact
    [CIERA abstract; section 4.6, Figure 10].
  * [CIERA Appendix A, Algorithm 1] sender: split, per-block change test,
    bitmap, payload of changed exponents; receiver: update the exponent cache
    for changed blocks, then merge.
  * [CIERA section 3.2] payload model S_{s+m} + S_bm + q*S_e with
    S_b = ceil(N/B) blocks and S_bm = ceil(S_b/8) bitmap bytes; compression is
    applied only to shards with a positive latency gain.

Readings where the pages leave the step open (each is listed with its reason
in the design notes of the repository):
  R1  change detection compares each exponent with the cached one exactly (the
      pages hash whole blocks; the exact compare is what the 128-bit hash
      approximates).
  R2  the changed exponents travel as (u32 shard-local index, u8 exponent)
      records in ascending index order, not entropy-coded.
  R3  bitmap bit b (byte b//8, bit b%8, least significant first) is set when
      block b holds at least one changed exponent; the bitmap is omitted when
      nothing changed.
  R4  sign|mantissa bytes: bf16 -> one byte (sign in bit 7, mantissa in bits
      6..0); fp32 -> three little-endian bytes of (sign << 23 | mantissa);
      fp16 (IEEE binary16: 1 sign, 5 exponent, 10 mantissa bits) -> the 11-bit
      value (sign << 10 | mantissa) of every element, packed back to back into
      one bit stream, least significant bit first: value i occupies bits
      [11i, 11i + 11), so 8 values fill 11 bytes and the section is
      ceil(11n/8) bytes.  The cache holds the 5-bit fp16 exponent in a byte.
  R5  a 64-byte little-endian header (layout in ``HEADER_FIELDS``).
  R6  the gain subtracts all codec costs; the link term is linear in bytes.
  R7  the plan's change rate is the element change fraction (ppm).
  R8  a stream is COMPRESSED only when strictly shorter than the raw stream.
  R9  decoding a RAW stream still refreshes the cache from the raw values.
  R12 row-sharding: rank r holds floor(R/W) + [r < R mod W] consecutive rows.

Parity status: split/join, lengths, cache update and encode/decode round trip
are pinned by exhaustive and closed-form tests; the byte layout (R2-R5) is
pinned by hand-derived known-answer streams of the written format; the plan is
pinned by a hand-computed decision table.  None of the byte layout is fixed by
the pages themselves.
"""
from __future__ import annotations

import struct
from typing import List, Optional, Sequence, Tuple

import numpy as np

# ------------------------------------------------------------------ constants

HEADER_BYTES = 64
MAGIC = b"CIER"
VERSION = 1
BF16 = 1
FP32 = 2
FP16 = 3
MODE_RAW = 0
MODE_COMPRESSED = 1
MODE_BLOCK = 2                     # the block-hash variant (R26-R28)
PATCH_BYTES = 5                    # u32 index + u8 exponent

# decode status bits
ST_MAGIC = 1       # bad magic or version
ST_FIELD = 2       # dtype / block size / n / offset / rank / world / mode mismatch
ST_LENGTH = 4      # total_len or n_changed inconsistent, or larger than the slot
ST_PATCH = 8       # a patch index >= n, or indices not strictly ascending
ST_BITMAP = 16     # bitmap disagrees with the patch list (unspecified if ST_PATCH), or
                   # (block variant) its set bits are not n_changed or a tail bit is set

# (name, byte offset, struct code) -- little-endian
HEADER_FIELDS = [
    ("magic", 0, "4s"), ("version", 4, "<H"), ("dtype", 6, "B"), ("mode", 7, "B"),
    ("block_size", 8, "<I"), ("reserved0", 12, "<I"), ("n", 16, "<Q"),
    ("n_changed", 24, "<Q"), ("total_len", 32, "<Q"), ("offset", 40, "<Q"),
    ("rank", 48, "<I"), ("world", 52, "<I"), ("reserved1", 56, "<Q"),
]


def elem_bytes(dtype: int) -> int:
    """e: bytes per value (16-bit bf16 and fp16, 32-bit fp32) [CIERA 3.2: S = N*b/8]."""
    return {BF16: 2, FP32: 4, FP16: 2}[dtype]


def sm_bits(dtype: int) -> int:
    """Sign|mantissa bits per value (R4): everything but the exponent bits."""
    return {BF16: 8, FP32: 24, FP16: 11}[dtype]


def sm_bytes(dtype: int) -> int:
    """k: sign|mantissa bytes per value of the byte-aligned types (bf16, fp32)."""
    return {BF16: 1, FP32: 3}[dtype]


def sm_section_bytes(n: int, dtype: int) -> int:
    """Bytes of the sign|mantissa section of n values: ceil(n * bits / 8) (R4)."""
    return -(-n * sm_bits(dtype) // 8)


def int_dtype(dtype: int):
    return {BF16: np.uint16, FP32: np.uint32, FP16: np.uint16}[dtype]


# -------------------------------------------------------- field split / merge
# [CIERA 3.1] "splits each weight value into exponent bits and sign-plus-mantissa
# bits".  Bit positions are those of IEEE-754 binary32 and of bfloat16 (binary32
# with the low 16 mantissa bits dropped): sign | 8 exponent bits | mantissa; and
# of IEEE-754 binary16: sign | 5 exponent bits | 10 mantissa bits.

# (exponent shift = mantissa bits, exponent mask, sign bit position)
_LAYOUT = {BF16: (7, 0xFF, 15), FP32: (23, 0xFF, 31), FP16: (10, 0x1F, 15)}


def exponent_field(u: np.ndarray, dtype: int) -> np.ndarray:
    shift, emask, _ = _LAYOUT[dtype]
    u = np.asarray(u).astype(np.uint32)
    return ((u >> shift) & emask).astype(np.uint8)


def sign_mantissa_field(u: np.ndarray, dtype: int) -> np.ndarray:
    """bf16 -> sign<<7 | mantissa(7);  fp32 -> sign<<23 | mantissa(23);
    fp16 -> sign<<10 | mantissa(10)."""
    shift, _, sbit = _LAYOUT[dtype]
    u = np.asarray(u).astype(np.uint32)
    return ((u >> sbit) << shift) | (u & ((1 << shift) - 1))


def join_fields(sm: np.ndarray, ex: np.ndarray, dtype: int) -> np.ndarray:
    """Inverse of the split: Merge(exponent, sign|mantissa) [CIERA Alg. 1, receiver]."""
    shift, _, sbit = _LAYOUT[dtype]
    sm = np.asarray(sm).astype(np.uint32)
    ex = np.asarray(ex).astype(np.uint32)
    u = ((sm >> shift) << sbit) | (ex << shift) | (sm & ((1 << shift) - 1))
    return u.astype(int_dtype(dtype))


def pack_sm(sm: np.ndarray, dtype: int) -> np.ndarray:
    """Pack sign|mantissa values (R4): k little-endian bytes each for bf16 and
    fp32; for fp16 an LSB-first bit stream of 11-bit values."""
    sm = np.asarray(sm).astype(np.uint32)
    if dtype == BF16:
        return sm.astype(np.uint8)
    if dtype == FP16:
        bits = (sm[:, None] >> np.arange(11, dtype=np.uint32)[None, :]) & 1   # bit j of value i
        return np.packbits(bits.astype(np.uint8).reshape(-1), bitorder="little")
    b = np.stack([sm & 0xFF, (sm >> 8) & 0xFF, (sm >> 16) & 0xFF], axis=1)
    return b.astype(np.uint8).reshape(-1)


def unpack_sm(b: np.ndarray, dtype: int, n: Optional[int] = None) -> np.ndarray:
    """Inverse of pack_sm; fp16 needs the value count n."""
    b = np.asarray(b, dtype=np.uint8)
    if dtype == BF16:
        return b.astype(np.uint32)
    if dtype == FP16:
        bits = np.unpackbits(b, bitorder="little")[:11 * n].reshape(n, 11).astype(np.uint32)
        return (bits << np.arange(11, dtype=np.uint32)[None, :]).sum(axis=1).astype(np.uint32)
    t = b.reshape(-1, 3).astype(np.uint32)
    return t[:, 0] | (t[:, 1] << 8) | (t[:, 2] << 16)


# ------------------------------------------------------------------ sharding

def shard(rows: int, cols: int, world: int, rank: int) -> Tuple[int, int]:
    """(element offset, element count) of rank's row shard (R12).

    ZeRO-3 style even partition of a row-major tensor: rank r holds
    floor(R/W) + [r < R mod W] consecutive rows."""
    q, rem = divmod(rows, world)
    rows_before = rank * q + min(rank, rem)
    my_rows = q + (1 if rank < rem else 0)
    return rows_before * cols, my_rows * cols


# ------------------------------------------------------------------- lengths
# [CIERA 3.2] S_b = ceil(N/B) blocks, S_bm = ceil(S_b/8) bitmap bytes.

def n_blocks(n: int, block_size: int) -> int:
    return -(-n // block_size)


def bitmap_bytes(n: int, block_size: int) -> int:
    return -(-n_blocks(n, block_size) // 8)


def raw_len(n: int, dtype: int) -> int:
    return HEADER_BYTES + n * elem_bytes(dtype)


def comp_len(n: int, n_changed: int, dtype: int, block_size: int) -> int:
    """Header + all sign|mantissa bytes (+ bitmap + 5-byte patches if anything changed)."""
    base = HEADER_BYTES + sm_section_bytes(n, dtype)
    if n_changed == 0:
        return base
    return base + bitmap_bytes(n, block_size) + PATCH_BYTES * n_changed


# ------------------------------------------------------------------- header

def pack_header(**f) -> bytes:
    out = bytearray(HEADER_BYTES)
    for name, off, code in HEADER_FIELDS:
        val = f.get(name, MAGIC if name == "magic" else 0)
        struct.pack_into(code, out, off, val)
    return bytes(out)


def parse_header(buf) -> dict:
    b = bytes(np.asarray(buf, dtype=np.uint8)[:HEADER_BYTES])
    if len(b) < HEADER_BYTES:
        raise ValueError("stream shorter than its header")
    return {name: struct.unpack_from(code, b, off)[0] for name, off, code in HEADER_FIELDS}


# -------------------------------------------------------------- cache update

def cache_update(w: np.ndarray, dtype: int) -> np.ndarray:
    """ExpCache <- exponents of the given (full) tensor [CIERA 3.1; Alg. 1 state]."""
    return exponent_field(np.asarray(w).reshape(-1), dtype)


# -------------------------------------------------------------------- encode

def encode(x: np.ndarray, cache_slice: np.ndarray, dtype: int, block_size: int,
           compress: bool, offset: int = 0, rank: int = 0, world: int = 1) -> np.ndarray:
    """Sender side of one Allgather for one shard [CIERA 3.1, Alg. 1 sender].

    x            -- the shard as integer bit patterns (uint16 for bf16, uint32 fp32)
    cache_slice  -- uint8 exponents cached for the same positions last iteration
    compress     -- the plan's decision (a RAW stream is written when 0)
    Returns the whole stream (header included) as a uint8 array of total_len bytes.
    """
    x = np.ascontiguousarray(np.asarray(x).reshape(-1)).astype(int_dtype(dtype))
    cache_slice = np.asarray(cache_slice, dtype=np.uint8).reshape(-1)
    n = x.size
    if cache_slice.size != n:
        raise ValueError("cache slice and shard differ in length")
    if n >= 1 << 32:
        raise ValueError("a shard holds fewer than 2^32 values (u32 patch indices)")
    # 1. split
    ex = exponent_field(x, dtype)
    sm = sign_mantissa_field(x, dtype)
    # 2. change detection, per element (R1)
    changed = ex != cache_slice
    idx = np.nonzero(changed)[0]
    n_changed = int(idx.size)
    # 3. lengths and mode (R8)
    c_len = comp_len(n, n_changed, dtype, block_size)
    r_len = raw_len(n, dtype)
    mode = MODE_COMPRESSED if (compress and c_len < r_len) else MODE_RAW
    total = c_len if mode == MODE_COMPRESSED else r_len
    hdr = pack_header(version=VERSION, dtype=dtype, mode=mode, block_size=block_size,
                      n=n, n_changed=n_changed, total_len=total, offset=offset,
                      rank=rank, world=world)
    out = np.zeros(total, dtype=np.uint8)
    out[:HEADER_BYTES] = np.frombuffer(hdr, dtype=np.uint8)
    if mode == MODE_RAW:
        le = np.dtype(int_dtype(dtype)).newbyteorder("<")
        out[HEADER_BYTES:] = x.astype(le).view(np.uint8)
        return out
    # 4. sign|mantissa bytes of every value
    pos = HEADER_BYTES
    out[pos:pos + sm_section_bytes(n, dtype)] = pack_sm(sm, dtype)
    pos += sm_section_bytes(n, dtype)
    if n_changed == 0:
        return out
    # 5. bitmap: one bit per block of B values that holds a change (R3)
    nbm = bitmap_bytes(n, block_size)
    bm = np.zeros(nbm, dtype=np.uint8)
    blocks = np.unique(idx // block_size)
    np.bitwise_or.at(bm, blocks // 8, (1 << (blocks % 8)).astype(np.uint8))
    out[pos:pos + nbm] = bm
    pos += nbm
    # 6. changed exponents as (index, exponent) records, ascending (R2)
    rec = np.zeros((n_changed, PATCH_BYTES), dtype=np.uint8)
    rec[:, 0:4] = idx.astype("<u4").view(np.uint8).reshape(n_changed, 4)
    rec[:, 4] = ex[idx]
    out[pos:pos + PATCH_BYTES * n_changed] = rec.reshape(-1)
    return out


# -------------------------------------------------------------------- decode

def _check_header(s: np.ndarray, dtype: int, block_size: int, n: int, offset: int,
                  rank: int, world: int, coded: bool = False) -> Tuple[int, Optional[dict]]:
    """Header and length validation of one received stream; (status bits,
    header).  Mode 3 is accepted only for a tensor declared coded (R35)."""
    if s.size < HEADER_BYTES:
        return ST_LENGTH, None
    h = parse_header(s)
    if h["magic"] != MAGIC or h["version"] != VERSION:
        return ST_MAGIC, None
    if (h["dtype"] != dtype or h["block_size"] != block_size or h["n"] != n
            or h["offset"] != offset or h["rank"] != rank or h["world"] != world
            or h["mode"] not in ((MODE_RAW, MODE_COMPRESSED, MODE_BLOCK, MODE_CODED) if coded
                                 else (MODE_RAW, MODE_COMPRESSED, MODE_BLOCK))):
        return ST_FIELD, None
    p = h["n_changed"]
    if p > (n_blocks(n, block_size) if h["mode"] == MODE_BLOCK else n) or h["total_len"] > s.size:
        return ST_LENGTH, None
    if h["mode"] == MODE_CODED:  # R33: the chunk table gives the length, checked per chunk
        base = HEADER_BYTES + sm_section_bytes(n, dtype)
        ok = (h["total_len"] == base if p == 0
              else h["total_len"] >= coded_comp_len(n, p, dtype, block_size, 0))
        return (0, h) if ok else (ST_LENGTH, None)
    if h["mode"] == MODE_RAW:
        want = raw_len(n, dtype)
    elif h["mode"] == MODE_COMPRESSED:
        want = comp_len(n, p, dtype, block_size)
    else:
        want = block_comp_len(n, p, dtype, block_size)
    if h["total_len"] != want:
        return ST_LENGTH, None
    return 0, h


def decode_stream(s: np.ndarray, dtype: int, block_size: int, n: int, offset: int,
                  rank: int, world: int, cache_slice: np.ndarray, coded: bool = False):
    """Receiver side for one stream [CIERA 3.1, Alg. 1 receiver].  coded: the
    tensor is declared to carry mode-3 streams (R35).

    Returns (values or None, new cache slice or None, status bits)."""
    s = np.asarray(s, dtype=np.uint8)
    st, h = _check_header(s, dtype, block_size, n, offset, rank, world, coded)
    if st:
        return None, None, st
    pos = HEADER_BYTES
    if h["mode"] == MODE_RAW:
        le = np.dtype(int_dtype(dtype)).newbyteorder("<")
        x = s[pos:pos + n * elem_bytes(dtype)].view(le).astype(int_dtype(dtype))
        return x, exponent_field(x, dtype), 0          # R9
    sms = sm_section_bytes(n, dtype)
    sm = unpack_sm(s[pos:pos + sms], dtype, n)
    pos += sms
    ex = np.array(cache_slice, dtype=np.uint8, copy=True)   # previous exponents
    if h["mode"] == MODE_BLOCK:
        return _decode_blocks(s, pos, h["n_changed"], n, block_size, sm, ex, dtype)
    if h["mode"] == MODE_CODED:
        return _decode_coded(s, pos, h, n, block_size, sm, ex, dtype)
    p = h["n_changed"]
    if p > 0:
        nbm = bitmap_bytes(n, block_size)
        bm = s[pos:pos + nbm]
        pos += nbm
        rec = s[pos:pos + PATCH_BYTES * p].reshape(p, PATCH_BYTES)
        idx = np.ascontiguousarray(rec[:, 0:4]).view("<u4").reshape(-1).astype(np.int64)
        val = rec[:, 4]
        if np.any(idx >= n) or np.any(np.diff(idx) <= 0):
            st |= ST_PATCH
        ok = idx < n
        # bitmap must mark exactly the blocks that hold a patch (tail bits zero)
        want = np.zeros(nbm, dtype=np.uint8)
        blocks = np.unique(idx[ok] // block_size)
        np.bitwise_or.at(want, blocks // 8, (1 << (blocks % 8)).astype(np.uint8))
        if not np.array_equal(want, bm):
            st |= ST_BITMAP
        ex[idx[ok]] = val[ok]                            # replace changed exponents
    return join_fields(sm, ex, dtype), ex, st


def decode(streams: Sequence[np.ndarray], rows: int, cols: int, dtype: int,
           block_size: int, world: int, cache_full: np.ndarray,
           out_full: Optional[np.ndarray] = None, coded: bool = False):
    """Rebuild the full tensor from all W ranks' streams and update the cache.

    streams[r] is rank r's receive slot (at least total_len bytes).  Returns
    (full tensor as integer bit patterns, updated cache, OR of status bits).
    Shards whose stream fails the header/length checks are left untouched."""
    N = rows * cols
    cache = np.array(cache_full, dtype=np.uint8, copy=True).reshape(-1)
    out = (np.zeros(N, dtype=int_dtype(dtype)) if out_full is None
           else np.array(out_full, copy=True).reshape(-1))
    status = 0
    for r in range(world):
        off, n = shard(rows, cols, world, r)
        x, ex, st = decode_stream(streams[r], dtype, block_size, n, off, r, world,
                                  cache[off:off + n], coded)
        status |= st
        if x is None:
            continue
        out[off:off + n] = x
        cache[off:off + n] = ex
    return out, cache, status


# ---------------------------------------------------------------------- plan
# [CIERA 3.2] g_i = Comm(S^i) - [Comm(S_{s+m} + S_bm + q_i S_e) + T_hash + T_cmp + T_decmp];
# keep the shard only if g_i > 0.  With pipelining, T_hash and T_cmp are off the
# critical path.  Comm is linear in bytes (alpha cancels); every quantity is an
# integer and every division floors, in the order written (R6, R7).

DEFAULT_COST = dict(link_bytes_per_us=8000,         # ~8 GB/s cross-node AllGather bus BW [CIERA 4.1]
                    hbm_bytes_per_us=5_600_000,     # 70% of 8 TB/s HBM3E
                    fixed_ns=5000,
                    overlap_encode=1)


def plan(rows: int, cols: int, dtype: int, block_size: int, world: int,
         change_ppm: int, cost: Optional[dict] = None) -> dict:
    c = dict(DEFAULT_COST)
    if cost:
        c.update(cost)
    e = elem_bytes(dtype)
    _, n = shard(rows, cols, world, 0)                 # the largest shard
    raw = raw_len(n, dtype)
    p_hat = (change_ppm * n + 999_999) // 1_000_000    # ceil
    comp = comp_len(n, p_hat, dtype, block_size)
    res = dict(raw_stream_bytes=raw, max_stream_bytes=raw, cache_bytes=rows * cols,
               expected_changed=p_hat)
    if comp >= raw:
        res.update(compress=0, expected_stream_bytes=raw, gain_ns=0)
        return res
    save = (raw - comp) * (world - 1) * 1000 // c["link_bytes_per_us"]
    dec = c["fixed_ns"] + world * (comp + n + n + n * e) * 1000 // c["hbm_bytes_per_us"]
    enc = 0 if c["overlap_encode"] else (
        c["fixed_ns"] + (n * e + n + comp) * 1000 // c["hbm_bytes_per_us"])
    gain = save - dec - enc
    compress = 1 if gain > 0 else 0
    res.update(compress=compress, expected_stream_bytes=comp if compress else raw, gain_ns=gain)
    return res


# ------------------------------------------------------------------ selection
# [CIERA 3.2] Among the shards with a positive gain g_i, rank them by g_i / M_i
# (gain per byte of exponent cache) in descending order and select them until
# the cache budget is exhausted.  Readings: M_i is the cache this design holds
# for the tensor (one byte per value of the full tensor, the plan's
# cache_bytes); equal ratios keep the input order; the selection stops at the
# first ranked shard whose cache no longer fits in what is left (R25).

def select(gains: Sequence[int], cache_bytes: Sequence[int], budget: int) -> List[int]:
    """compress flags (0/1) per tensor: the benefit-driven selection."""
    from fractions import Fraction
    cand = [i for i in range(len(gains)) if gains[i] > 0]

    def ratio(i):  # a shard with no cache costs nothing: it ranks first
        return Fraction(gains[i], cache_bytes[i]) if cache_bytes[i] > 0 else float("inf")

    ranked = sorted(cand, key=lambda i: ratio(i), reverse=True)  # sorted() is stable
    # reverse=True keeps equal keys in their input order as well
    out = [0] * len(gains)
    used = 0
    for i in ranked:
        if used + cache_bytes[i] > budget:
            break
        out[i] = 1
        used += cache_bytes[i]
    return out


# ------------------------------------------------------- block-hash variant
# [CIERA 3.1; Appendix A, Algorithm 1] as the pages publish it: the sender
# keeps a 128-bit hash of every block's exponents (HashCache, 16 bytes per
# block instead of the exponents themselves), built from two independent
# 64-bit SplitMix64 hashes [ref. 22 of the page]; a block whose hash differs
# from the cached one is marked in the bitmap, its hash replaces the cached
# one, and its exponents travel whole.  Readings:
#   R26 the 64-bit hash of a block: its exponent bytes (one per value) as
#       little-endian 8-byte words w_j, the last one zero-padded;
#       H_s = mix64((sum_j mix64(w_j ^ (s + (j + 1) * GAMMA)) + L) mod 2^64)
#       with L the block's byte length, mix64 SplitMix64's output function and
#       GAMMA its increment; the position-keyed sum can be formed in parallel
#       over a block's words (the word-wise hashing of the page's ref. [23]).
#       The two halves use the seeds HASH_SEEDS.
#   R27 the payload (the pages ANS-code it with a closed library): the
#       exponent bytes of each changed block, in block order, B bytes per
#       block, the last block zero-padded to B.  The stream is
#       header (mode 2, n_changed = changed blocks) | sign|mantissa |
#       [bitmap | payload] if any block changed; BLOCK only when strictly
#       shorter than RAW (R8).
#   R28 the receiver: cached exponents, the changed blocks replaced from the
#       payload, merged with the sign|mantissa bits; bitmap set bits other
#       than n_changed, or a set bit past the last block, is ST_BITMAP.
# Parity unpinned against the pages: the hash's constants and word layout
# (the pages name SplitMix64 but give no construction); the hash is sender
# state and never travels, and the pins check that it marks exactly the blocks
# whose exponents changed.

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15                           # SplitMix64 increment
HASH_SEEDS = (0x243F6A8885A308D3, 0x13198A2E03707344)  # digits of pi, for two independent halves


def mix64(z: int) -> int:
    """SplitMix64's output function (Steele, Lea and Flood; 64-bit variant)."""
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def block_hash64(b: bytes, seed: int) -> int:
    """R26: one 64-bit hash of a block's exponent bytes."""
    L = len(b)
    padded = bytes(b) + bytes(-L % 8)
    acc = 0
    for j in range(len(padded) // 8):
        w = int.from_bytes(padded[8 * j:8 * j + 8], "little")
        acc = (acc + mix64(w ^ ((seed + (j + 1) * GAMMA) & MASK64))) & MASK64
    return mix64((acc + L) & MASK64)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    """mix64 elementwise on uint64 arrays (numpy's uint64 products wrap mod 2^64)."""
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def block_hashes(ex: np.ndarray, block_size: int) -> np.ndarray:
    """The 128-bit hash of every block of an exponent array: (blocks, 2) uint64;
    block_hash64 of each block, evaluated for all blocks at once."""
    ex = np.asarray(ex, dtype=np.uint8).reshape(-1)
    n = ex.size
    nb = n_blocks(n, block_size)
    out = np.zeros((nb, 2), dtype=np.uint64)
    if nb == 0:
        return out
    wpb = block_size // 8                           # words per block (B >= 64)
    padded = np.zeros(nb * block_size, dtype=np.uint8)
    padded[:n] = ex
    words = padded.view("<u8").reshape(nb, wpb).astype(np.uint64)
    L = np.full(nb, block_size, dtype=np.uint64)
    L[-1] = n - (nb - 1) * block_size
    nwords = (L + np.uint64(7)) // np.uint64(8)      # words that belong to each block
    j1 = np.arange(1, wpb + 1, dtype=np.uint64)      # j + 1
    valid = np.arange(wpb)[None, :] < nwords[:, None].astype(np.int64)
    with np.errstate(over="ignore"):
        for h, seed in enumerate(HASH_SEEDS):
            keys = np.uint64(seed) + j1 * np.uint64(GAMMA)
            terms = np.where(valid, _mix64_np(words ^ keys[None, :]), np.uint64(0))
            acc = terms.sum(axis=1, dtype=np.uint64)
            out[:, h] = _mix64_np(acc + L)
    return out


def hash_seed(x: np.ndarray, dtype: int, block_size: int) -> np.ndarray:
    """HashCache of a shard: the hash of each block's exponents (after warmup)."""
    return block_hashes(exponent_field(np.asarray(x).reshape(-1), dtype), block_size)


def block_comp_len(n: int, n_changed_blocks: int, dtype: int, block_size: int) -> int:
    """Header + sign|mantissa (+ bitmap + B bytes per changed block)."""
    base = HEADER_BYTES + sm_section_bytes(n, dtype)
    if n_changed_blocks == 0:
        return base
    return base + bitmap_bytes(n, block_size) + n_changed_blocks * block_size


def encode_block(x: np.ndarray, hashes: np.ndarray, dtype: int, block_size: int, compress: bool,
                 offset: int = 0, rank: int = 0, world: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Sender side of the block-hash variant [CIERA Alg. 1 sender]: returns the
    stream and the updated HashCache of the shard."""
    x = np.ascontiguousarray(np.asarray(x).reshape(-1)).astype(int_dtype(dtype))
    n = x.size
    nb = n_blocks(n, block_size)
    hashes = np.asarray(hashes, dtype=np.uint64).reshape(nb, 2)
    ex = exponent_field(x, dtype)
    sm = sign_mantissa_field(x, dtype)
    new = block_hashes(ex, block_size)
    changed = np.nonzero(np.any(new != hashes, axis=1))[0]
    c = int(changed.size)
    c_len = block_comp_len(n, c, dtype, block_size)
    r_len = raw_len(n, dtype)
    mode = MODE_BLOCK if (compress and c_len < r_len) else MODE_RAW
    total = c_len if mode == MODE_BLOCK else r_len
    hdr = pack_header(version=VERSION, dtype=dtype, mode=mode, block_size=block_size,
                      n=n, n_changed=c, total_len=total, offset=offset, rank=rank, world=world)
    out = np.zeros(total, dtype=np.uint8)
    out[:HEADER_BYTES] = np.frombuffer(hdr, dtype=np.uint8)
    if mode == MODE_RAW:
        le = np.dtype(int_dtype(dtype)).newbyteorder("<")
        out[HEADER_BYTES:] = x.astype(le).view(np.uint8)
        return out, new
    pos = HEADER_BYTES
    out[pos:pos + sm_section_bytes(n, dtype)] = pack_sm(sm, dtype)
    pos += sm_section_bytes(n, dtype)
    if c == 0:
        return out, new
    nbm = bitmap_bytes(n, block_size)
    bm = np.zeros(nbm, dtype=np.uint8)
    np.bitwise_or.at(bm, changed // 8, (1 << (changed % 8)).astype(np.uint8))
    out[pos:pos + nbm] = bm
    pos += nbm
    for j, k in enumerate(changed):          # whole blocks, the last zero-padded (R27)
        blk = ex[k * block_size:(k + 1) * block_size]
        out[pos + j * block_size:pos + j * block_size + blk.size] = blk
    return out, new


def _decode_blocks(s, pos, c, n, block_size, sm, ex, dtype):
    """R28: replace the changed blocks of the cached exponents and merge."""
    st = 0
    if c > 0:
        nb = n_blocks(n, block_size)
        nbm = bitmap_bytes(n, block_size)
        bm = s[pos:pos + nbm]
        payload = s[pos + nbm:pos + nbm + c * block_size]
        bits = np.unpackbits(bm, bitorder="little")
        if np.any(bits[nb:]) or int(bits[:nb].sum()) != c:
            st |= ST_BITMAP
        for j, k in enumerate(np.nonzero(bits[:nb])[0][:c]):
            L = min(block_size, n - k * block_size)
            ex[k * block_size:k * block_size + L] = payload[j * block_size:j * block_size + L]
    return join_fields(sm, ex, dtype), ex, st



# ---------------------------------------- entropy-coded patches (mode 3)
# [CIERA 3.1] the sender compresses the changed exponents with ANS; [CIERA
# Alg. 1] ANS-encode on the sender, ANS-decode on the receiver.  The pages
# name the coder (ANS, through a vendor library) but not its model or layout;
# this mode codes each element patch -- the gap since the previous change and
# the new exponent relative to the cached one -- with range ANS (Duda,
# "Asymmetric numeral systems", 2009/2013), interleaved over several coder
# states (Giesen, "Interleaved entropy coders", 2014).  Readings:
#   R29 the shard is cut into chunks of 4096 values from value 0 (the last may
#       be shorter); each chunk is coded on its own, so chunks decode in
#       parallel.
#   R30 a chunk with c changes is sent as rANS data when c <= 1024 and the
#       data is shorter than the dense form, else dense: the chunk's new
#       exponent bytes, zero-padded to a multiple of 4.  A chunk without
#       changes sends nothing.
#   R31 rANS data: L = min(64, ceil(c/4)) coder states; change j (in index
#       order) goes to state j mod L.  Per change four symbols, in decode
#       order: the gap bucket b = bit length of (gap + 1), where gap = index
#       minus previous index minus 1 (the first change of a chunk counts from
#       the chunk start, previous index -1); the b - 1 bits of gap + 1 below
#       its leading one, as a uniform symbol; the exponent class (+1, -1, +2,
#       -2, ..., +7, -7 modulo 256, or escape); for an escape the new exponent
#       itself as a uniform 8-bit symbol.  Gap buckets use the frequencies of
#       a geometric gap distribution with p = c / chunk length, computed in
#       32-bit fixed point (``gap_bucket_freqs``); exponent classes use a
#       fixed table (``DELTA_FREQ``).  Both sum to 2^12.
#   R32 32-bit states kept in [2^16, 2^32), renormalized by 16-bit words.  The
#       decoder goes through the changes L at a time and through the four
#       symbols of each change as four sub-steps; after each sub-step every
#       state below 2^16, in state order, takes the next word.  The encoder
#       runs the same sub-steps backwards, each state starting at 2^16, and
#       its final states open the chunk data: states (u32 each) | words (u16
#       each) | a zero word when their number is odd.
#   R33 stream (mode 3): header | sign|mantissa | [bitmap | zero bytes to a
#       multiple of 4 from the stream start | chunk table | chunk data] if
#       anything changed.  Chunk table: per chunk, two u32 -- the changes and
#       the data bytes of this and all earlier chunks.  Mode 3 only when
#       strictly shorter than RAW (R8).
#   R34 decode checks: a chunk table entry that goes backwards, exceeds the
#       chunk length or the data, has a byte count not a multiple of 4, data
#       without changes or changes without data, rANS data shorter than its
#       states or longer than the dense form, or a last entry other than
#       (n_changed, data bytes) is
#       ST_LENGTH and the chunk is not decoded.  Within a chunk, a change past
#       its end, an exponent wider than the field, words missing or left
#       over, a final state other than 2^16, or dense data whose differences
#       from the cache number other than c, is ST_PATCH.  The bitmap verdict
#       is unspecified alongside ST_LENGTH or ST_PATCH.
#   R35 a receiver accepts mode 3 only for a tensor it declared coded (the
#       decode of such tensors carries the rANS decoder); otherwise the mode
#       is a field mismatch (ST_FIELD).
# Parity unpinned against the pages (they fix no ANS model or layout); the
# pins are the rANS definition's closed forms, its entropy bound, per-state
# independence, and round trips.

MODE_CODED = 3
CHUNK = 4096
CODED_MAX_PATCHES = 1024
RANS_LOW = 1 << 16
RANS_SCALE = 12
GAP_BUCKETS = 13
DELTA_FREQ = (2032, 2032) + (2,) * 12 + (8,)
DELTA_ESCAPE = 14


def pad4(v: int) -> int:
    return (v + 3) & ~3


def n_chunks(n: int) -> int:
    return (n + CHUNK - 1) // CHUNK


def chunk_length(n: int, k: int) -> int:
    return min(CHUNK, n - k * CHUNK)


def rans_lanes(c: int) -> int:
    return min(64, (c + 3) // 4)


def gap_bucket_freqs(c: int, length: int) -> List[int]:
    """R31: frequencies (sum 2^12) of gap buckets 1..13 for a chunk of
    `length` values holding c changes.  With q = 1 - c/length in 32-bit fixed
    point, S[i] ~ q^(2^i - 1) is the chance that a gap is at least 2^i - 1;
    bucket b (gaps 2^(b-1) - 1 .. 2^b - 2) gets S[b-1] - S[b], the last bucket
    the rest.  Each frequency is that share of 2^12, at least 1; the largest
    (first of equals) absorbs the rounding."""
    q = ((length - c) << 32) // length
    Q = [q]
    for _ in range(GAP_BUCKETS - 2):
        Q.append((Q[-1] * Q[-1]) >> 32)           # q^(2^i)
    S = [1 << 32]
    for i in range(GAP_BUCKETS - 1):
        S.append((S[-1] * Q[i]) >> 32)            # q^(2^(i+1) - 1)
    share = [S[b - 1] - S[b] for b in range(1, GAP_BUCKETS)] + [S[GAP_BUCKETS - 1]]
    f = [max(1, v >> (32 - RANS_SCALE)) for v in share]
    top = f.index(max(f))
    f[top] += (1 << RANS_SCALE) - sum(f)
    return f


def _cum(freqs: Sequence[int]) -> List[int]:
    out, t = [], 0
    for v in freqs:
        out.append(t)
        t += v
    return out


def delta_class(old: int, new: int) -> int:
    """R31: +1 -> 0, -1 -> 1, +2 -> 2, -2 -> 3, ..., +7 -> 12, -7 -> 13 (mod 256), else escape (14)."""
    d = (new - old) & 0xFF
    for k in range(1, 8):
        if d == k:
            return 2 * (k - 1)
        if d == 256 - k:
            return 2 * (k - 1) + 1
    return DELTA_ESCAPE


def class_delta(cls: int) -> int:
    k = cls // 2 + 1
    return k if cls % 2 == 0 else 256 - k


def rans_encode(substeps: Sequence[Sequence[Tuple[int, int, int, int]]], lanes: int):
    """rANS encoder over interleaved states (R32).  substeps lists, in decode
    order, the symbols of each sub-step as (state, start, frequency, scale
    bits), the frequencies of a symbol set summing to 2^scale.  The encoder
    visits them backwards; before coding symbol s into state x it writes the
    low 16 bits of x out while x >= f_s * 2^(32 - scale), then
    x <- floor(x / f_s) * 2^scale + (x mod f_s) + start_s.  Returns the final
    states and the words in the order the decoder reads them."""
    x = [RANS_LOW] * lanes
    emitted = []
    for sub in reversed(substeps):
        out = []
        for lane, start, freq, scale in sub:
            if x[lane] >= freq << (32 - scale):
                out.append((lane, x[lane] & 0xFFFF))
                x[lane] >>= 16
            x[lane] = ((x[lane] // freq) << scale) + x[lane] % freq + start
        emitted.append([w for _, w in sorted(out)])   # read in state order
    words = [w for sub in reversed(emitted) for w in sub]
    return x, words


def _chunk_symbols(offs: Sequence[int], olds: Sequence[int], news: Sequence[int], length: int):
    """R31: the chunk's changes as four sub-steps per round of L changes."""
    c = len(offs)
    L = rans_lanes(c)
    gf = gap_bucket_freqs(c, length)
    gc, dc = _cum(gf), _cum(DELTA_FREQ)
    subs = []
    prev = -1
    for t in range((c + L - 1) // L):
        A, Bs, C, D = [], [], [], []
        for lane in range(L):
            j = t * L + lane
            if j >= c:
                break
            g = offs[j] - prev - 1
            prev = offs[j]
            b = (g + 1).bit_length()
            A.append((lane, gc[b - 1], gf[b - 1], RANS_SCALE))
            if b > 1:
                Bs.append((lane, (g + 1) - (1 << (b - 1)), 1, b - 1))
            cls = delta_class(olds[j], news[j])
            C.append((lane, dc[cls], DELTA_FREQ[cls], RANS_SCALE))
            if cls == DELTA_ESCAPE:
                D.append((lane, news[j], 1, 8))
        subs += [A, Bs, C, D]
    return subs, L


def encode_chunk(ex_chunk: np.ndarray, cache_chunk: np.ndarray) -> bytes:
    """R30-R32: the data of one chunk (new exponents and cached ones)."""
    ex_chunk = np.asarray(ex_chunk, dtype=np.uint8)
    cache_chunk = np.asarray(cache_chunk, dtype=np.uint8)
    length = int(ex_chunk.size)
    offs = np.nonzero(ex_chunk != cache_chunk)[0]
    c = int(offs.size)
    if c == 0:
        return b""
    dense = bytes(ex_chunk) + bytes(pad4(length) - length)
    if c > CODED_MAX_PATCHES:
        return dense
    subs, L = _chunk_symbols([int(v) for v in offs], [int(cache_chunk[v]) for v in offs],
                             [int(ex_chunk[v]) for v in offs], length)
    states, words = rans_encode(subs, L)
    data = struct.pack(f"<{L}I", *states) + struct.pack(f"<{len(words)}H", *words)
    if len(words) % 2:
        data += bytes(2)
    return data if len(data) < len(dense) else dense


def coded_comp_len(n: int, n_changed: int, dtype: int, block_size: int, data_bytes: int) -> int:
    """R33: header + sign|mantissa (+ bitmap, padding, chunk table and data)."""
    base = HEADER_BYTES + sm_section_bytes(n, dtype)
    if n_changed == 0:
        return base
    return pad4(base + bitmap_bytes(n, block_size)) + 8 * n_chunks(n) + data_bytes


def encode_coded(x: np.ndarray, cache_slice: np.ndarray, dtype: int, block_size: int,
                 compress: bool, offset: int = 0, rank: int = 0, world: int = 1) -> np.ndarray:
    """Sender side with entropy-coded patches [CIERA 3.1 ANS-encode; R29-R33]."""
    x = np.ascontiguousarray(np.asarray(x).reshape(-1)).astype(int_dtype(dtype))
    cache_slice = np.asarray(cache_slice, dtype=np.uint8).reshape(-1)
    n = x.size
    if cache_slice.size != n:
        raise ValueError("cache slice and shard differ in length")
    ex = exponent_field(x, dtype)
    sm = sign_mantissa_field(x, dtype)
    changed = ex != cache_slice
    P = int(np.count_nonzero(changed))
    chunks = [encode_chunk(ex[k * CHUNK:k * CHUNK + chunk_length(n, k)],
                           cache_slice[k * CHUNK:k * CHUNK + chunk_length(n, k)]) for k in range(n_chunks(n))] if P else []
    c_len = coded_comp_len(n, P, dtype, block_size, sum(len(d) for d in chunks))
    r_len = raw_len(n, dtype)
    mode = MODE_CODED if (compress and c_len < r_len) else MODE_RAW
    total = c_len if mode == MODE_CODED else r_len
    hdr = pack_header(version=VERSION, dtype=dtype, mode=mode, block_size=block_size,
                      n=n, n_changed=P, total_len=total, offset=offset, rank=rank, world=world)
    out = np.zeros(total, dtype=np.uint8)
    out[:HEADER_BYTES] = np.frombuffer(hdr, dtype=np.uint8)
    if mode == MODE_RAW:
        le = np.dtype(int_dtype(dtype)).newbyteorder("<")
        out[HEADER_BYTES:] = x.astype(le).view(np.uint8)
        return out
    pos = HEADER_BYTES
    out[pos:pos + sm_section_bytes(n, dtype)] = pack_sm(sm, dtype)
    pos += sm_section_bytes(n, dtype)
    if P == 0:
        return out
    nbm = bitmap_bytes(n, block_size)
    blocks = np.unique(np.nonzero(changed)[0] // block_size)
    bm = np.zeros(nbm, dtype=np.uint8)
    np.bitwise_or.at(bm, blocks // 8, (1 << (blocks % 8)).astype(np.uint8))
    out[pos:pos + nbm] = bm
    pos = pad4(pos + nbm)
    cc = cb = 0
    table = bytearray()
    for k, d in enumerate(chunks):
        cc += int(np.count_nonzero(changed[k * CHUNK:k * CHUNK + chunk_length(n, k)]))
        cb += len(d)
        table += struct.pack("<II", cc, cb)
    out[pos:pos + len(table)] = np.frombuffer(bytes(table), dtype=np.uint8)
    pos += len(table)
    data = b"".join(chunks)
    out[pos:pos + len(data)] = np.frombuffer(data, dtype=np.uint8)
    return out


def rans_decode_chunk(data: bytes, c: int, length: int, cache_chunk: np.ndarray, emask: int):
    """R31-R32, R34: decode one chunk's rANS data.  Returns (offsets, new
    exponents, status); changes past the chunk or with an exponent wider than
    the field are flagged and left out."""
    L = rans_lanes(c)
    x = list(struct.unpack_from(f"<{L}I", data, 0))
    nw = (len(data) - 4 * L) // 2
    words = struct.unpack_from(f"<{nw}H", data, 4 * L)
    st = 0
    ptr = 0
    gf = gap_bucket_freqs(c, length)
    gc, dc = _cum(gf), _cum(DELTA_FREQ)

    def find(cum, freqs, slot):
        s = 0
        while s + 1 < len(cum) and cum[s + 1] <= slot:
            s += 1
        return s

    def renorm():
        nonlocal ptr, st
        for lane in range(L):
            if x[lane] < RANS_LOW:
                if ptr < nw:
                    w = words[ptr]
                else:
                    w = 0
                    st |= ST_PATCH
                ptr += 1
                x[lane] = ((x[lane] << 16) | w) & 0xFFFFFFFF

    offs, news = [], []
    prev = -1
    for t in range((c + L - 1) // L):
        act = [lane for lane in range(L) if t * L + lane < c]
        b, g, cls, esc = {}, {}, {}, {}
        for lane in act:                      # gap bucket
            slot = x[lane] & ((1 << RANS_SCALE) - 1)
            s = find(gc, gf, slot)
            x[lane] = gf[s] * (x[lane] >> RANS_SCALE) + slot - gc[s]
            b[lane] = s + 1
        renorm()
        for lane in act:                      # bits of gap + 1 below the leading one
            k = b[lane] - 1
            v = x[lane] & ((1 << k) - 1)
            x[lane] >>= k
            g[lane] = (1 << k) + v - 1
        renorm()
        for lane in act:                      # exponent class
            slot = x[lane] & ((1 << RANS_SCALE) - 1)
            s = find(dc, DELTA_FREQ, slot)
            x[lane] = DELTA_FREQ[s] * (x[lane] >> RANS_SCALE) + slot - dc[s]
            cls[lane] = s
        renorm()
        for lane in act:                      # escaped exponent
            if cls[lane] == DELTA_ESCAPE:
                esc[lane] = x[lane] & 0xFF
                x[lane] >>= 8
        renorm()
        for lane in act:                      # indices in change order
            idx = prev + g[lane] + 1
            prev = idx
            if idx >= length:
                st |= ST_PATCH
                continue
            new = esc[lane] if cls[lane] == DELTA_ESCAPE else (int(cache_chunk[idx]) + class_delta(cls[lane])) & 0xFF
            if new > emask:
                st |= ST_PATCH
                continue
            offs.append(idx)
            news.append(new)
    if ptr + (ptr & 1) != nw or any(v != RANS_LOW for v in x):
        st |= ST_PATCH
    return offs, news, st


def _decode_coded(s, pos, h, n, block_size, sm, ex, dtype):
    """R33-R34: receiver side of mode 3 (ex holds the cached exponents)."""
    P = h["n_changed"]
    st = 0
    if P == 0:
        return join_fields(sm, ex, dtype), ex, st
    emask = _LAYOUT[dtype][1]
    nbm = bitmap_bytes(n, block_size)
    bm = s[pos:pos + nbm]
    tpos = pad4(pos + nbm)
    nch = n_chunks(n)
    dpos = tpos + 8 * nch
    D = h["total_len"] - dpos
    table = struct.unpack_from(f"<{2 * nch}I", bytes(s[tpos:dpos]))
    touched = np.zeros(n, dtype=bool)
    pc = pb = 0
    for k in range(nch):
        cc, cb = table[2 * k], table[2 * k + 1]
        length = chunk_length(n, k)
        c, nbytes = cc - pc, cb - pb
        bad = (cc < pc or cb < pb or cb > D or c > length or nbytes % 4 != 0 or (c == 0) != (nbytes == 0)
               or (k == nch - 1 and (cc != P or cb != D)))
        if not bad and c > 0 and nbytes != pad4(length) and (nbytes < 4 * rans_lanes(c) or nbytes > pad4(length)):
            bad = True                          # rANS data holds its states and is shorter than dense
        if bad:
            st |= ST_LENGTH
        elif c > 0:
            data = bytes(s[dpos + pb:dpos + cb])
            base = k * CHUNK
            old = ex[base:base + length].copy()
            if nbytes == pad4(length):          # dense
                new = np.frombuffer(data[:length], dtype=np.uint8)
                if np.any(new > emask) or int(np.count_nonzero(new != old)) != c:
                    st |= ST_PATCH
                touched[base:base + length] = new != old
                ex[base:base + length] = new
            else:
                offs, news, e = rans_decode_chunk(data, c, length, old, emask)
                st |= e
                for o, v in zip(offs, news):
                    touched[base + o] = True
                    ex[base + o] = v
        pc, pb = cc, cb                         # the next chunk starts where this entry says
    want = np.zeros(nbm, dtype=np.uint8)
    blocks = np.unique(np.nonzero(touched)[0] // block_size)
    np.bitwise_or.at(want, blocks // 8, (1 << (blocks % 8)).astype(np.uint8))
    if not np.array_equal(want, bm):
        st |= ST_BITMAP
    return join_fields(sm, ex, dtype), ex, st
