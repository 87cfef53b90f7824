"""Seeded random and extreme arguments to the host-only entry points of the C
ABI -- ciera_plan, ciera_plan_batch, ciera_select, ciera_shard and the two
scratch-size queries -- without a GPU.  Every call returns one of the header's
status codes; where it succeeds, plan and shard agree with the oracle
[CIERA 3.2], plan_batch with plan per tensor, and the scratch sizes are
deterministic.  None of these entry points touches the device: the item
pointers are checked for null and alignment only, so fake aligned addresses
are safe here (the prepare and launch calls, which copy to the device, are
not called)."""
import ctypes
import random

import pytest

from oracle import ciera_oracle as O

L = pytest.importorskip("lossless_weight_compression_amd")
from lossless_weight_compression_amd import _binding as B  # noqa: E402

STATUS = {0, 1, 2, 3, 4}
EDGE = [0, 1, 2, 3, 7, 15, 16, 17, 63, 64, 4095, 4096, 4097, 8192, 65536, 1 << 20, (1 << 31) - 1, 1 << 31,
        1 << 32, (1 << 32) + 1, 1 << 40, (1 << 63) - 1, (1 << 64) - 1]


class Args:
    def __init__(self, seed):
        self.r = random.Random(seed)

    def num(self, bits=64):
        r = self.r
        v = r.choice(EDGE) if r.random() < 0.7 else r.getrandbits(r.choice([8, 16, 32, 64]))
        return v & ((1 << bits) - 1)

    def tensor(self):
        r = self.r
        if r.random() < 0.6:  # mostly valid shapes
            return B.Tensor(r.randint(0, 5000), r.randint(1, 5000), r.choice([1, 2, 3]),
                            r.choice([64, 128, 256, 512, 1024, 2048, 4096]), r.randint(1, 16), r.choice([0, 0, 1]))
        return B.Tensor(self.num(), self.num(), r.choice([0, 1, 2, 3, 4, 255, 1 << 31]),
                        r.choice([0, 1, 2, 16, 63, 64, 128, 512, 1536, 4096, 8192, 1 << 16, 1 << 31]),
                        r.choice([0, 1, 2, 3, 16, 64, 1024, 1 << 20, 1 << 31]), r.choice([0, 1, 2, 3, 0xFFFFFFFF]))

    def ptr(self):
        r = self.r
        if r.random() < 0.7:
            return 0x7F0000000000 + 256 * r.randrange(1 << 20)  # aligned, never dereferenced here
        return r.choice([0, 16, 0x1001, 0x7F0000000008])


def _status(st):
    assert st in STATUS, st
    return st


def test_plan_and_shard_random_arguments():
    a, lib = Args(1), B._lib
    n_ok = 0
    for _ in range(3000):
        t = a.tensor()
        ppm = a.num(32)
        p = B.Plan()
        st = _status(lib.ciera_plan(ctypes.byref(t), ppm, None, ctypes.byref(p)))
        if st == 0:
            n_ok += 1
            q = O.plan(t.rows, t.cols, t.dtype, t.block_size, t.world, ppm)
            assert (p.compress, p.raw_stream_bytes, p.expected_stream_bytes, p.gain_ns) == \
                (q["compress"], q["raw_stream_bytes"], q["expected_stream_bytes"], q["gain_ns"])
        rank = a.r.choice([0, 1, 2, a.num(32)])
        off, n = ctypes.c_uint64(), ctypes.c_uint64()
        st = _status(lib.ciera_shard(ctypes.byref(t), rank, ctypes.byref(off), ctypes.byref(n)))
        if st == 0:
            assert (off.value, n.value) == O.shard(t.rows, t.cols, t.world, rank)
    assert n_ok > 1000


def test_plan_batch_random_arguments():
    a, lib = Args(2), B._lib
    for _ in range(400):
        k = a.r.choice([0, 1, 2, 5, 33])
        ts = (B.Tensor * max(k, 1))(*[a.tensor() for _ in range(k)])
        pp = (ctypes.c_uint32 * max(k, 1))(*[a.num(32) for _ in range(k)])
        out = (B.Plan * max(k, 1))()
        st = _status(lib.ciera_plan_batch(ts, pp, k, None, out))
        first = 0
        for i in range(k):
            p = B.Plan()
            s = lib.ciera_plan(ctypes.byref(ts[i]), pp[i], None, ctypes.byref(p))
            if s != 0:
                first = s
                break
            assert bytes(p) == bytes(out[i])
        assert st == first


def test_select_random_plans():
    a, lib = Args(3), B._lib
    for _ in range(500):
        k = a.r.choice([0, 1, 2, 7, 40])
        plans = (B.Plan * max(k, 1))()
        gains, caches = [], []
        for i in range(k):
            g = a.r.choice([0, 1, -1, 5, 10 ** 6, -(10 ** 9), (1 << 62), a.r.randrange(-(1 << 40), 1 << 40)])
            c = a.r.choice([0, 1, 2, 1000, 1 << 30, 1 << 40, a.r.randrange(0, 1 << 40)])
            plans[i].gain_ns, plans[i].cache_bytes = g, c
            gains.append(g)
            caches.append(c)
        budget = a.num(64)
        out = (ctypes.c_uint32 * max(k, 1))()
        assert _status(lib.ciera_select(plans, k, budget, out)) == 0
        assert [out[i] for i in range(k)] == O.select(gains, caches, budget)


def test_scratch_sizes_random_items():
    a, lib = Args(4), B._lib
    keep = []
    for _ in range(1500):
        k = a.r.choice([0, 1, 2, 5, 40])
        enc = (B.EncodeItem * max(k, 1))()
        dec = (B.DecodeItem * max(k, 1))()
        for i in range(k):
            enc[i].t, enc[i].rank, enc[i].compress = a.tensor(), a.r.choice([0, 1, 2, 15, a.num(32)]), \
                a.r.choice([0, 1, 2, 3, 4, 99])
            enc[i].shard, enc[i].cache_full, enc[i].stream = a.ptr(), a.ptr(), a.ptr()
            enc[i].stream_capacity = a.num() if a.r.random() < 0.4 else 1 << 40
            t = a.tensor()
            dec[i].t, dec[i].streams, dec[i].out_full, dec[i].cache_full = t, a.ptr(), a.ptr(), a.ptr()
            dec[i].slot_bytes = a.num() if a.r.random() < 0.4 else 16 * a.r.randrange(1, 1 << 22)
            if a.r.random() < 0.3 and 0 < t.world <= 4096:  # a host array of one pointer per rank
                rs = (ctypes.c_void_p * t.world)(*[a.ptr() for _ in range(t.world)])
                keep.append(rs)
                dec[i].rank_streams = ctypes.cast(rs, ctypes.c_void_p)
        for f, items in ((lib.ciera_encode_scratch_bytes, enc), (lib.ciera_decode_scratch_bytes, dec)):
            b1, b2 = ctypes.c_uint64(), ctypes.c_uint64()
            s1 = _status(f(items, k, ctypes.byref(b1)))
            s2 = f(items, k, ctypes.byref(b2))
            assert s1 == s2 and (s1 != 0 or b1.value == b2.value)
        keep = keep[-64:]
