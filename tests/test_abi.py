"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-only logic (plan, shard, argument checks) agrees with
the oracle.  No device call is made here."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import ciera_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ciera.h")

L = pytest.importorskip("lossless_weight_compression_amd")


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ciera_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(L._binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", L._binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ciera_\w+)", out))
    missing = set(declared_symbols()) - exported
    assert not missing, missing
    lib = ctypes.CDLL(L._binding.LIB_PATH)
    for s in declared_symbols():
        assert hasattr(lib, s)


def test_abi_version_and_strings():
    assert L.ciera_abi_version() == 4
    assert L.ciera_status_str(0) == "ok"
    assert "buffer" in L.ciera_status_str(2)


def _rand_tensors(seed, count):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        rows = int(rng.choice([0, 1, 7, 448, 1024, 2048, 7168, int(rng.integers(1, 100000))]))
        cols = int(rng.choice([1, 3, 256, 1024, 2048, int(rng.integers(1, 5000))]))
        yield (rows, cols, int(rng.choice([1, 2, 3])), int(2 ** rng.integers(6, 13)),
               int(rng.choice([1, 2, 4, 8, 16, 64, int(rng.integers(1, 200))])))


def test_plan_parity_with_oracle():
    rng = np.random.default_rng(3)
    for rows, cols, dt, B, W in _rand_tensors(1, 3000):
        ppm = int(rng.choice([0, 1, 100, 1000, 10000, 50000, 190000, 300000, 1000000,
                              int(rng.integers(0, 1000001))]))
        cost = dict(link_bytes_per_us=int(rng.choice([8000, 153000, 1, 10 ** 7])),
                    hbm_bytes_per_us=int(rng.choice([5_600_000, 8_000_000, 1000])),
                    fixed_ns=int(rng.choice([0, 5000, 100000])),
                    overlap_encode=int(rng.integers(0, 2)))
        p = L.ciera_plan(L.Tensor(rows, cols, dt, B, W), ppm, L.CostModel(**cost))
        q = O.plan(rows, cols, dt, B, W, ppm, cost)
        assert p.compress == q["compress"]
        assert p.raw_stream_bytes == q["raw_stream_bytes"] == p.max_stream_bytes
        assert p.expected_stream_bytes == q["expected_stream_bytes"]
        assert p.gain_ns == q["gain_ns"]
        assert p.expected_changed == q["expected_changed"]
        assert p.cache_bytes == rows * cols


def test_plan_defaults_match_hand_table():
    from tests.test_oracle_brute_plan import PLAN_TABLE
    for rows, cols, dt, W, ppm, compress, expected, gain in PLAN_TABLE:
        p = L.ciera_plan(L.Tensor(rows, cols, dt, 512, W), ppm)
        assert (p.compress, p.expected_stream_bytes, p.gain_ns) == (compress, expected, gain)


def test_shard_parity_with_oracle():
    for rows, cols, dt, B, W in _rand_tensors(2, 500):
        t = L.Tensor(rows, cols, dt, B, W)
        for r in range(W):
            assert L.ciera_shard(t, r) == O.shard(rows, cols, W, r)


def test_argument_errors_are_synchronous():
    bad = [L.Tensor(4, 4, 4, 512, 1), L.Tensor(4, 4, 0, 512, 1), L.Tensor(4, 4, 1, 500, 1), L.Tensor(4, 4, 1, 32, 1),
           L.Tensor(4, 4, 1, 8192, 1), L.Tensor(4, 4, 1, 512, 0)]
    for t in bad:
        with pytest.raises(L.CieraError) as e:
            L.ciera_plan(t, 100)
        assert e.value.code == 1
    with pytest.raises(L.CieraError):
        L.ciera_plan(L.Tensor(4, 4, 1, 512, 1), 1_000_001)
    # u32 patch indices: the largest shard must hold fewer than 2^32 values
    for t in (L.Tensor(1 << 20, 1 << 12, 1, 512, 1), L.Tensor((1 << 21) + 1, 1 << 12, 1, 512, 2)):
        with pytest.raises(L.CieraError) as e:
            L.ciera_plan(t, 100)
        assert e.value.code == 3
    assert L.ciera_plan(L.Tensor((1 << 20) - 1, 1 << 12, 1, 512, 1), 100).raw_stream_bytes == \
        64 + 2 * ((1 << 20) - 1) * (1 << 12)
    with pytest.raises(L.CieraError) as e:
        L.ciera_shard(L.Tensor(4, 4, 1, 512, 2), 2)
    assert e.value.code == 1
    with pytest.raises(L.CieraError) as e:
        L.ciera_plan(L.Tensor(1 << 33, 1 << 20, 1, 512, 1), 100)
    assert e.value.code == 3


def test_encode_decode_validation_without_device():
    t = L.Tensor(64, 64, 1, 512, 2)
    good = dict(shard=0x10000, cache_full=0x20000, stream_buf=0x30000)

    def enc(**kw):
        a = dict(good, **kw)
        it = L.encode_item(t, kw.get("rank", 0), 1, a["shard"], a["cache_full"], a["stream_buf"],
                           kw.get("cap", 64 + 32 * 64 * 2))
        need = L.ciera_encode_scratch_bytes([it])
        L.ciera_encode([it], kw.get("scratch", 0x40000), kw.get("sbytes", need), stream=0)

    cases = [(dict(shard=0x10008), 1), (dict(stream_buf=0x30004), 1), (dict(stream_buf=0), 1),
             (dict(cap=64 + 32 * 64 * 2 - 1), 2), (dict(scratch=0x40010), 1), (dict(sbytes=16), 2),
             (dict(rank=2), 1)]
    for kw, code in cases:
        with pytest.raises(L.CieraError) as e:
            enc(**kw)
        assert e.value.code == code, kw
    # decode
    d = L.decode_item(t, 0x30000, 64 + 32 * 64 * 2 + 16, 0x50000, 0x20000)
    need = L.ciera_decode_scratch_bytes([d])
    for kw, code in [(dict(streams=0x30008), 1), (dict(slot_bytes=40), 1), (dict(slot_bytes=48), 2),
                     (dict(out_full=0x50002), 1)]:
        a = dict(streams=0x30000, slot_bytes=64 + 32 * 64 * 2 + 16, out_full=0x50000)
        a.update(kw)
        di = L.decode_item(t, a["streams"], a["slot_bytes"], a["out_full"], 0x20000)
        with pytest.raises(L.CieraError) as e:
            L.ciera_decode([di], 0x60000, 0x40000, need, stream=0)
        assert e.value.code == code, kw
    with pytest.raises(L.CieraError):
        L.ciera_decode([d], 0, 0x40000, need, stream=0)          # no status word


def test_overlapping_buffers_are_rejected_without_device():
    """Encode: the stream written must not overlap the shard or the cache
    slice it reads; decode: the rebuilt values, the cache and the W slots are
    disjoint.  Checked on the host before any device call (fake addresses)."""
    t = L.Tensor(64, 64, 1, 512, 2)               # shards of 32x64 bf16: 4096 B; stream <= 4160 B
    cap = 64 + 32 * 64 * 2

    def enc(shard, cache_full, stream):
        it = L.encode_item(t, 1, 1, shard, cache_full, stream, cap)
        L.ciera_encode([it], 0x900000, L.ciera_encode_scratch_bytes([it]), stream=0)

    for shard, cache, stream in [(0x10000, 0x20000, 0x10000 + 4096 - 16),   # stream ends in the shard
                                 (0x10000 + 4096 - 16, 0x20000, 0x10000),   # shard starts in the stream
                                 (0x10000, 0x30000 - 2048 - 16, 0x30000)]:  # rank 1's cache slice
        with pytest.raises(L.CieraError) as e:
            enc(shard, cache, stream)
        assert e.value.code == 1, (hex(shard), hex(cache), hex(stream))
    slot = cap + 16
    d_ok = dict(streams=0x100000, out_full=0x200000, cache=0x300000)
    bad = [dict(out_full=0x100000 + 2 * slot - 16),     # values start in the last slot
           dict(cache=0x200000 + 2 * 4096 - 1),         # cache starts in the values' last byte
           dict(cache=0x100000 - 4096 + 1),              # cache ends in the first slot
           dict(out_full=0x300000 - 8192 + 16)]          # values end in the cache
    for kw in bad:
        a = dict(d_ok, **kw)
        di = L.decode_item(t, a["streams"], slot, a["out_full"], a["cache"])
        with pytest.raises(L.CieraError) as e:
            L.ciera_decode([di], 0x800000, 0x900000, L.ciera_decode_scratch_bytes([di]), stream=0)
        assert e.value.code == 1, kw


def test_plan_batch_equals_plan_per_tensor():
    """ciera_plan_batch gives exactly ciera_plan for every tensor (random shapes,
    types, worlds, block sizes and change rates, default and custom cost
    models); a rejected tensor gives its status; null arrays are invalid."""
    import random
    rng = random.Random(5)
    ts, ppm = [], []
    for _ in range(400):
        dt = rng.choice([L.CIERA_BF16, L.CIERA_FP32, L.CIERA_FP16])
        ts.append(L.Tensor(rng.randint(1, 4000), rng.randint(1, 9000), dt, 1 << rng.randint(6, 12),
                           rng.randint(1, 64)))
        ppm.append(rng.choice([0, 1, 100, 10_000, 100_000, 300_000, 1_000_000]))
    for cost in (None, L.CostModel(12_000, 4_000_000, 3_000, 0)):
        got = L.ciera_plan_batch(ts, ppm, cost)
        want = [L.ciera_plan(t, p, cost) for t, p in zip(ts, ppm)]
        assert [g.as_dict() for g in got] == [w.as_dict() for w in want]
        pb = L.PlanBatch(ts, ppm, cost)
        assert [p.as_dict() for p in pb.run()] == [w.as_dict() for w in want]
    bad = ts[:3] + [L.Tensor(4, 4, 9, 512, 1)] + ts[3:5]
    with pytest.raises(L.CieraError) as e:
        L.ciera_plan_batch(bad, 100)
    assert e.value.code == 1
    with pytest.raises(ValueError):
        L.PlanBatch(ts[:3], [1, 2])
    assert L._binding._lib.ciera_plan_batch(None, None, 0, None, None) == 0
    assert L._binding._lib.ciera_plan_batch(None, None, 2, None, None) == 1


def test_rank_stream_pointers_without_device():
    """Decode items whose W streams sit in W separate buffers (rank_streams):
    exactly one of streams and rank_streams; every rank pointer non-null and
    16-byte aligned; no rank's range may overlap the rebuilt values or the
    cache; the scratch holds 8 bytes per rank pointer.  All refused on the host
    before any device call (fake addresses)."""
    t = L.Tensor(64, 64, 1, 512, 2)               # 2 ranks of 32x64 bf16
    slot = 64 + 32 * 64 * 2 + 16
    ranks = [0x100000, 0x140000]
    ok = dict(streams=None, rank_streams=ranks, out_full=0x200000, cache=0x300000)
    bad = [dict(streams=0x180000),                          # both layouts
           dict(rank_streams=None),                         # neither
           dict(rank_streams=[0x100000, 0x140008]),         # misaligned rank pointer
           dict(rank_streams=[0x100000, 0]),                # null rank pointer
           dict(rank_streams=[0x100000, 0x200000 + 8192 - 16]),   # rank 1 ends past the values' start
           dict(rank_streams=[0x300000 - slot + 16, 0x140000])]   # rank 0 runs into the cache
    for kw in bad:
        a = dict(ok, **kw)
        di = L.decode_item(t, a["streams"], slot, a["out_full"], a["cache"], rank_streams=a["rank_streams"])
        with pytest.raises(L.CieraError) as e:
            L.ciera_decode([di], 0x800000, 0x900000, L.ciera_decode_scratch_bytes([di]), stream=0)
        assert e.value.code == 1, kw
    with pytest.raises(ValueError):
        L.decode_item(t, None, slot, 0x200000, 0x300000, rank_streams=[0x100000])
    # 8 bytes per rank pointer, past the descriptors
    t16 = L.Tensor(64, 64, 1, 512, 16)
    slot16 = 64 + 4 * 64 * 2 + 16
    d_slots = L.decode_item(t16, 0x100000, slot16, 0x200000, 0x300000)
    d_ranks = L.decode_item(t16, None, slot16, 0x200000, 0x300000,
                            rank_streams=[0x400000 + 0x1000 * r for r in range(16)])
    base = L.ciera_decode_scratch_bytes([d_slots] * 40)
    more = L.ciera_decode_scratch_bytes([d_ranks] * 40)
    assert more - base >= 40 * 16 * 8 and (more - base) % 256 == 0


def test_scratch_sizes_grow_with_work():
    t1 = L.Tensor(2048, 1024, 1, 512, 16)
    it = L.encode_item(t1, 0, 1, 0x10000, 0x20000, 0x30000, 1 << 30)
    a = L.ciera_encode_scratch_bytes([it])
    b = L.ciera_encode_scratch_bytes([it] * 64)
    assert 0 < a < b and a % 256 == 0
    d = L.decode_item(t1, 0x30000, 1 << 20, 0x50000, 0x20000)
    assert L.ciera_decode_scratch_bytes([d] * 10) > L.ciera_decode_scratch_bytes([d])


def test_coded_patch_arguments_without_device():
    """compress = 3 needs the tensor flag CIERA_TENSOR_CODED; unknown flag bits
    are invalid; a coded shard of 2^31 values or more is unsupported (its chunk
    table's u32 byte counts could overflow)."""
    with pytest.raises(L.CieraError) as e:
        L.ciera_plan(L.Tensor(4, 4, 1, 512, 1, flags=2), 100)
    assert e.value.code == 1
    assert L.ciera_plan(L.Tensor(4, 4, 1, 512, 1, flags=L.CIERA_TENSOR_CODED), 100).raw_stream_bytes == 64 + 32

    def scratch(t, compress):
        return L.ciera_encode_scratch_bytes([L.encode_item(t, 0, compress, 0x10000, 0x20000, 0x30000,
                                                           64 + 2 * t.rows * t.cols)])

    flag = L.CIERA_TENSOR_CODED
    assert scratch(L.Tensor(2048, 1024, 1, 512, 1, flags=flag), 3) > 0          # 256 tiles of 8192 values
    assert scratch(L.Tensor(2049, 1024, 1, 512, 1, flags=flag), 3) > 0          # 257 tiles: scanned first
    assert scratch(L.Tensor((1 << 31) - 1, 1, 1, 512, 1, flags=flag), 3) > 0
    with pytest.raises(L.CieraError) as e:
        scratch(L.Tensor(1 << 31, 1, 1, 512, 1, flags=flag), 3)
    assert e.value.code == 3
    assert scratch(L.Tensor(2049, 1024, 1, 512, 1), 1) > 0                      # element patches: any size
    # coded tiles keep a 4096-byte region per chunk row plus 8 info words
    assert scratch(L.Tensor(8, 1024, 1, 512, 1, flags=flag), 3) >= scratch(L.Tensor(8, 1024, 1, 512, 1), 1) + 32
    it = L.encode_item(L.Tensor(64, 64, 1, 512, 2), 0, 3, 0x10000, 0x20000, 0x30000, 64 + 32 * 64 * 2)
    need = L.ciera_encode_scratch_bytes([it])
    with pytest.raises(L.CieraError) as e:       # no CIERA_TENSOR_CODED flag
        L.ciera_encode([it], 0x40000, need, stream=0)
    assert e.value.code == 1
    it = L.encode_item(L.Tensor(64, 64, 1, 512, 2, flags=flag), 0, 4, 0x10000, 0x20000, 0x30000, 64 + 32 * 64 * 2)
    with pytest.raises(L.CieraError) as e:       # compress beyond 3
        L.ciera_encode([it], 0x40000, need, stream=0)
    assert e.value.code == 1


def test_binding_rejects_tensors_it_would_misread():
    """A torch tensor handed to the binding must be contiguous, of the element
    type and count the call implies, and on a GPU; otherwise the library would
    read the wrong memory (a transposed weight encoded from its storage order).
    Checked before any device call."""
    import torch

    t = L.Tensor(64, 64, L.CIERA_BF16, 512, 2)          # rank 0: 32 x 64 values
    B = L._binding
    w = torch.zeros(64, 64, dtype=torch.bfloat16)
    cases = [
        (lambda: B._ptr(w.t(), "shard"), "not contiguous"),
        (lambda: L.encode_item(t, 0, 1, w[:32].t(), 0x20000, 0x30000, 8192), "not contiguous"),
        (lambda: L.encode_item(t, 0, 1, w[:32].view(torch.int16), 0x20000, 0x30000, 8192), "dtype"),
        (lambda: L.encode_item(t, 0, 1, w[:31], 0x20000, 0x30000, 8192), "elements"),
        (lambda: L.encode_item(t, 0, 1, w[:32], 0x20000, 0x30000, 8192), "not on a GPU"),
        (lambda: L.encode_item(t, 0, 1, 0x10000, torch.zeros(100, dtype=torch.uint8), 0x30000, 8192),
         "at least 4096"),
        (lambda: L.decode_item(t, 0x30000, 8208, torch.zeros(4095, dtype=torch.bfloat16), 0x20000), "elements"),
        (lambda: L.ciera_cache_update(t, w.to(torch.float32), 0x20000, stream=0), "dtype"),
        (lambda: L.ciera_hash_update(t, 1, w[32:].t(), 0x20000, stream=0), "not contiguous"),
    ]
    for call, msg in cases:
        with pytest.raises(ValueError, match=msg):
            call()
    assert B._ptr(None) is None and B._ptr(0x1234) == 0x1234


def test_noalloc_limits_without_device():
    """ciera_encode_noalloc refuses, before any device call, what its static
    scratch cannot hold or what needs a finishing kernel."""
    t = L.Tensor(64, 64, 1, 512, 2)
    it = L.encode_item(t, 0, 1, 0x10000, 0x20000, 0x30000, 64 + 32 * 64 * 2)
    for compress, code in ((2, 3), (4, 1)):
        bad = L.encode_item(t, 0, compress, 0x10000, 0x20000, 0x30000, 64 + 32 * 64 * 2)
        with pytest.raises(L.CieraError) as e:
            L.ciera_encode_noalloc([bad], stream=0)
        assert e.value.code == code
    big = L.Tensor(1 << 21, 1, 1, 512, 1)            # 256 tiles: needs a stash-free path, fits
    huge = L.Tensor((1 << 21) + 1, 1, 1, 512, 1)     # 257 tiles: would need a finishing kernel
    with pytest.raises(L.CieraError) as e:
        L.ciera_encode_noalloc([L.encode_item(huge, 0, 1, 0x10000, 0x20000, 0x40000000, 1 << 26)], stream=0)
    assert e.value.code == 3
    assert L.ciera_encode_scratch_bytes([L.encode_item(big, 0, 1, 0x10000, 0x20000, 0x40000000, 1 << 26)]) \
        < L._binding.CIERA_NOALLOC_SCRATCH_BYTES
    many = [it] * 9000                                # descriptors alone beyond 1 MiB
    assert L.ciera_encode_scratch_bytes(many) > L._binding.CIERA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(L.CieraError) as e:
        L.ciera_encode_noalloc(many, stream=0)
    assert e.value.code == 2
