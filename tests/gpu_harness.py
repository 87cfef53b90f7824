"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and compare byte for byte."""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from oracle import ciera_oracle as O

DT = {torch.bfloat16: O.BF16, torch.float32: O.FP32, torch.float16: O.FP16}
IV = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.float16: torch.int16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    """Integer bit patterns of a bf16/fp16/fp32 tensor as numpy uint16/uint32."""
    iv = t.detach().reshape(-1).view(IV[t.dtype]).cpu().numpy()
    return iv.view(np.uint32 if t.dtype == torch.float32 else np.uint16)


def header_total(slot: np.ndarray) -> int:
    return int(O.parse_header(slot)["total_len"])


class Case:
    """One layer (list of (rows, cols)) through encode of every rank + decode,
    on the GPU and in the oracle, from the same W0 (cache seed) and W1."""

    def __init__(self, shapes: Sequence[Tuple[int, int]], dtype: torch.dtype, world: int,
                 block_size: int = 512, change_ppm: int = 10_000):
        from lossless_weight_compression_amd.layer import LayerCodec
        self.shapes = list(shapes)
        self.dtype = dtype
        self.odt = DT[dtype]
        self.world = world
        self.B = block_size
        self.codec = LayerCodec(self.shapes, dtype, world, block_size, "cuda", change_ppm)

    def run(self, w0: List[torch.Tensor], w1: List[torch.Tensor], compress: Optional[Sequence[int]] = None,
            tensors: Optional[Sequence[int]] = None, edits=None, valid_edits_decode: bool = False) -> dict:
        """Seed the cache from w0, encode w1 for every rank (one batched call per
        rank), apply byte ``edits`` [(tensor, rank, offset, bytes)] to the
        streams on both sides, decode, and compare with the oracle.  ``tensors``
        limits the oracle comparison (all by default).  With
        ``valid_edits_decode``, edited streams that both sides decode with
        status 0 must also give the oracle's values and cache."""
        c = self.codec
        dev = [x.to("cuda").contiguous() for x in w0]
        c.seed_cache(dev)
        torch.cuda.synchronize()
        # the oracle seeds its own cache; the GPU's seed must equal it
        cache0 = [O.cache_update(to_np(w0[i]), self.odt) for i in range(len(self.shapes))]
        for i in range(len(self.shapes)):
            assert np.array_equal(c.cache_view(i).cpu().numpy(), cache0[i]), f"cache seed {i}"
        d1 = [x.to("cuda").contiguous() for x in w1]
        comp = compress if compress is not None else [p.compress for p in c.plans]
        for r in range(self.world):
            shards = []
            for i in range(len(self.shapes)):
                off, n = c.shard(i, r)
                shards.append(d1[i].reshape(-1)[off:off + n].clone())
            c.encode(r, shards, compress=comp)
        torch.cuda.synchronize()
        edits = list(edits or [])
        for (i, r, o, b) in edits:
            c.slot(i, r)[o:o + len(b)] = torch.tensor(list(b), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        slots = [[c.slot(i, r).cpu().numpy().copy() for r in range(self.world)]
                 for i in range(len(self.shapes))]
        st = c.decode()
        torch.cuda.synchronize()
        res = dict(status=int(st.item()), ostatus=0)
        which = range(len(self.shapes)) if tensors is None else tensors
        for i in which:
            rows, cols = self.shapes[i]
            x1 = to_np(w1[i])
            o_slots = []
            for r in range(self.world):
                off, n = O.shard(rows, cols, self.world, r)
                s = O.encode(x1[off:off + n], cache0[i][off:off + n], self.odt, self.B,
                             bool(comp[i]), off, r, self.world)
                got = slots[i][r][:s.size]
                if not edits:
                    assert np.array_equal(got, s), self._diff(i, r, got, s)
                pad = np.zeros(c.slot_bytes[i], dtype=np.uint8)
                pad[:s.size] = s
                o_slots.append(pad)
            for (ei, er, o, b) in edits:
                if ei == i:
                    o_slots[er][o:o + len(b)] = np.frombuffer(bytes(b), dtype=np.uint8)
            o_out, o_cache, o_st = O.decode(o_slots, rows, cols, self.odt, self.B, self.world, cache0[i])
            res["ostatus"] |= o_st
            if not edits:
                g_out = to_np(c.out_view(i))
                g_cache = c.cache_view(i).cpu().numpy()
                assert np.array_equal(g_out, o_out), f"tensor {i}: decoded values differ"
                assert np.array_equal(g_out, x1), f"tensor {i}: decode(encode(x)) != x"
                assert np.array_equal(g_cache, o_cache), f"tensor {i}: caches differ"
            elif valid_edits_decode and o_st == 0 and res["status"] == 0:
                assert np.array_equal(to_np(c.out_view(i)), o_out), f"tensor {i}: edited stream, values differ"
                assert np.array_equal(c.cache_view(i).cpu().numpy(), o_cache), f"tensor {i}: edited stream, caches differ"
        return res

    @staticmethod
    def _diff(i, r, got, want):
        bad = np.nonzero(got != want)[0]
        return (f"tensor {i} rank {r}: {bad.size} bytes differ, first at {bad[:8].tolist()} "
                f"got {got[bad[:8]].tolist()} want {want[bad[:8]].tolist()} (len {want.size})")
