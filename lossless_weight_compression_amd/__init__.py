"""CIERA exponent-reuse codec for MI355X (gfx950).

``_binding`` mirrors include/ciera.h (ciera_plan, ciera_select, ciera_shard, ciera_encode,
ciera_decode, ciera_cache_update, ...) over the in-tree libciera.so; ``layer``
holds a layer's caches, receive slots and outputs in flat device buffers.
Importing fails loudly when the library has not been built.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (Batch, CieraError, CostModel, DecodeItem, EncodeItem, Plan, PlanBatch, Tensor,  # noqa: F401
                       ciera_abi_version, ciera_cache_update, ciera_decode, ciera_decode_launch,
                       ciera_decode_launch_bounded, ciera_decode_prepare, ciera_decode_scratch_bytes, ciera_encode,
                       ciera_encode_noalloc,
                       ciera_encode_launch, ciera_encode_prepare, ciera_encode_scratch_bytes, ciera_hash_update,
                       ciera_plan, ciera_plan_batch, ciera_select, ciera_set_sync_polls, ciera_shard, ciera_status_str, decode_item,
                       encode_item)
