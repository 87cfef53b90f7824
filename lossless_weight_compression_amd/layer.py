"""A layer's worth of codec state on one GPU, laid out for HBM.

For a list of tensors sharded over W ranks this holds, in three flat device
buffers, what one rank keeps across iterations and receives each iteration:

  cache   -- one byte per value of every full tensor (the exponent cache)
  streams -- the receive buffer of the Allgather: per tensor, W slots of
             ``slot_bytes`` (the RAW length of the largest shard, rounded up to
             16 bytes); rank r's stream of tensor i sits in slot (i, r)
  out     -- the rebuilt full tensors

and issues one batched ``ciera_encode`` (a rank's shards of every tensor) or one
batched ``ciera_decode`` (every tensor from all W slots) per call.  torch is
used for device memory and streams only.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from . import _binding as B

TORCH_TO_CIERA = {torch.bfloat16: B.CIERA_BF16, torch.float32: B.CIERA_FP32, torch.float16: B.CIERA_FP16}
ELEM = {B.CIERA_BF16: 2, B.CIERA_FP32: 4, B.CIERA_FP16: 2}


def _align(x: int, a: int) -> int:
    return (x + a - 1) // a * a


class LayerCodec:
    def __init__(self, shapes: Sequence[Tuple[int, int]], dtype: torch.dtype, world: int,
                 block_size: int = 512, device="cuda", change_ppm: int = 10_000,
                 cost: Optional[B.CostModel] = None, with_out: bool = True,
                 cache: Optional[torch.Tensor] = None, cache_budget: Optional[int] = None,
                 coded: Optional[Sequence[bool]] = None):
        self.dtype = dtype
        self.cdtype = TORCH_TO_CIERA[dtype]
        self.e = ELEM[self.cdtype]
        self.world = world
        self.device = torch.device(device)
        coded = coded or [False] * len(shapes)  # tensors whose streams may be CODED
        self.tensors = [B.Tensor(r, c, self.cdtype, block_size, world, B.CIERA_TENSOR_CODED if k else 0)
                        for (r, c), k in zip(shapes, coded)]
        self.numel = [r * c for r, c in shapes]
        self.plans = [B.ciera_plan(t, change_ppm, cost) for t in self.tensors]
        if cache_budget is not None:  # benefit-driven selection: the rest is sent RAW
            for p, c in zip(self.plans, B.ciera_select(self.plans, cache_budget)):
                p.compress = c
        self.slot_bytes = [_align(p.max_stream_bytes, 16) for p in self.plans]
        # flat buffers with 256-byte aligned per-tensor regions
        self.cache_off, self.stream_off, self.out_off = [], [], []
        c = s = o = 0
        for i, n in enumerate(self.numel):
            self.cache_off.append(c)
            c += _align(n, 256)
            self.stream_off.append(s)
            s += _align(self.slot_bytes[i] * world, 256)
            self.out_off.append(o)
            o += _align(n * self.e, 256)
        if cache is not None:  # share another codec's cache (same shapes, same layout)
            assert cache.dtype == torch.uint8 and cache.numel() >= max(c, 256)
            self.cache = cache
        else:
            self.cache = torch.zeros(max(c, 256), dtype=torch.uint8, device=self.device)
        self.streams = torch.zeros(max(s, 256), dtype=torch.uint8, device=self.device)
        self.out = (torch.zeros(max(o, 256), dtype=torch.uint8, device=self.device)
                    if with_out else None)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        self._dec_items = [B.decode_item(t, self.streams.data_ptr() + self.stream_off[i], self.slot_bytes[i],
                                         (self.out.data_ptr() + self.out_off[i]) if with_out else None,
                                         self.cache.data_ptr() + self.cache_off[i])
                           for i, t in enumerate(self.tensors)]
        self.dec_scratch = torch.empty(max(B.ciera_decode_scratch_bytes(self._dec_items), 256),
                                       dtype=torch.uint8, device=self.device)
        self._dec_batch = None
        self._enc_scratch = None
        self._hashes = None

    # ------------------------------------------------------------------ views
    def shard(self, i: int, rank: int) -> Tuple[int, int]:
        return B.ciera_shard(self.tensors[i], rank)

    def cache_view(self, i: int) -> torch.Tensor:
        return self.cache[self.cache_off[i]:self.cache_off[i] + self.numel[i]]

    def slot(self, i: int, rank: int) -> torch.Tensor:
        a = self.stream_off[i] + rank * self.slot_bytes[i]
        return self.streams[a:a + self.slot_bytes[i]]

    def out_view(self, i: int) -> torch.Tensor:
        a = self.out_off[i]
        return self.out[a:a + self.numel[i] * self.e].view(self.dtype)

    # ------------------------------------------------------------------ calls
    def seed_cache(self, weights: Sequence[torch.Tensor], stream=None) -> None:
        """cache <- exponents of the given full tensors (exponent reuse switched on)."""
        for i, w in enumerate(weights):
            B.ciera_cache_update(self.tensors[i], w, self.cache.data_ptr() + self.cache_off[i], stream)

    def hash_cache(self, i: int, rank: int) -> torch.Tensor:
        """Sender state of the block-hash variant for (tensor i, rank): 16 bytes
        per block of the shard (allocated on first use)."""
        if self._hashes is None:
            self._hash_off, h = {}, 0
            for j, t in enumerate(self.tensors):
                for r in range(self.world):
                    _, n = self.shard(j, r)
                    self._hash_off[(j, r)] = h
                    h += _align(16 * (-(-n // t.block_size)), 256)
            self._hashes = torch.zeros(max(h, 256), dtype=torch.uint8, device=self.device)
        _, n = self.shard(i, rank)
        o = self._hash_off[(i, rank)]
        return self._hashes[o:o + 16 * (-(-n // self.tensors[i].block_size))]

    def share_hash_caches(self, other: "LayerCodec") -> None:
        """Use other's block-variant hash caches (same shapes), as `cache=` shares
        the exponent cache: two codecs that alternate iterations of one layer."""
        other.hash_cache(0, 0)
        self._hashes, self._hash_off = other._hashes, other._hash_off

    def seed_hashes(self, rank: int, shards: Sequence[torch.Tensor], stream=None) -> None:
        """The block-hash variant's hash caches of rank's shards (reuse switched on)."""
        for i, t in enumerate(self.tensors):
            B.ciera_hash_update(t, rank, shards[i], self.hash_cache(i, rank).data_ptr(), stream)

    def encode_items(self, rank: int, shards: Sequence[torch.Tensor],
                     compress: Optional[Sequence[int]] = None) -> List[B.EncodeItem]:
        """compress[i]: 0 RAW, 1 COMPRESSED (default: the plan's), 2 the block-hash
        variant, which reads and updates rank's hash cache of tensor i, 3
        entropy-coded patches (shards of fewer than 2^31 values)."""
        items = []
        for i, t in enumerate(self.tensors):
            c = self.plans[i].compress if compress is None else compress[i]
            a = self.stream_off[i] + rank * self.slot_bytes[i]
            state = (self.hash_cache(i, rank).data_ptr() if c == B.BLOCK
                     else self.cache.data_ptr() + self.cache_off[i])
            _, n = self.shard(i, rank)
            x = B._ptr(shards[i], f"shard of tensor {i}", self.dtype, n)
            items.append(B.EncodeItem(t, rank, c, x, state, self.streams.data_ptr() + a, self.slot_bytes[i]))
        return items

    def encode_scratch(self, items: Sequence[B.EncodeItem]) -> torch.Tensor:
        need = max(B.ciera_encode_scratch_bytes(items), 256)
        if self._enc_scratch is None or self._enc_scratch.numel() < need:
            self._enc_scratch = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._enc_scratch

    def encode(self, rank: int, shards: Sequence[torch.Tensor], stream=None,
               compress: Optional[Sequence[int]] = None, items=None) -> None:
        """Encode rank's shard of every tensor into its slots (one batched call)."""
        items = items if items is not None else self.encode_items(rank, shards, compress)
        B.ciera_encode(items, self.encode_scratch(items), stream=stream)

    def decode(self, stream=None, zero_status: bool = True, max_workgroups: int = 0) -> torch.Tensor:
        """Rebuild every tensor from its W slots and update the cache (one launch of
        the prepared decode batch; its tables are uploaded on the first call).
        max_workgroups > 0 bounds the decode's grid (ciera_decode_launch_bounded)."""
        if zero_status:
            self.status.zero_()
        if self._dec_batch is None:
            self._dec_batch = B.ciera_decode_prepare(self._dec_items, self.status, self.dec_scratch,
                                                     stream=stream)
        B.ciera_decode_launch_bounded(self._dec_batch, max_workgroups, stream=stream)
        return self.status

    def prepare_encode(self, rank: int, shards: Sequence[torch.Tensor],
                       compress: Optional[Sequence[int]] = None, stream=None) -> "PreparedEncode":
        """A prepared encode of rank's shards: tables uploaded once, each launch
        then only enqueues kernels (the shard buffers stay bound)."""
        items = self.encode_items(rank, shards, compress)
        scratch = torch.empty(max(B.ciera_encode_scratch_bytes(items), 256), dtype=torch.uint8,
                              device=self.device)
        return PreparedEncode(B.ciera_encode_prepare(items, scratch, stream=stream), scratch, list(shards))


class PreparedEncode:
    def __init__(self, batch: "B.Batch", scratch: torch.Tensor, keep: list):
        self.batch, self.scratch, self._keep = batch, scratch, keep

    def launch(self, stream=None) -> None:
        B.ciera_encode_launch(self.batch, stream=stream)
