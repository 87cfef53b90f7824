"""ctypes binding of libciera.so: same names as include/ciera.h, argument
marshalling only.  Every step of encode/decode runs in the HIP kernels; there
is no fallback -- importing this module fails if the library is not built."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_int, c_int64, c_uint32, c_uint64, c_void_p
from typing import List, Optional, Sequence, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libciera.so")

CIERA_BF16, CIERA_FP32, CIERA_FP16 = 1, 2, 3
RAW, COMPRESSED, BLOCK, CODED = 0, 1, 2, 3  # encode item `compress` values and stream modes
CIERA_TENSOR_CODED = 1  # Tensor.flags: the tensor's streams may be CODED
CIERA_OK, CIERA_ERR_INVALID_ARG, CIERA_ERR_BUFFER_TOO_SMALL, CIERA_ERR_UNSUPPORTED, CIERA_ERR_DEVICE = range(5)
CIERA_ST_MAGIC, CIERA_ST_FIELD, CIERA_ST_LENGTH, CIERA_ST_PATCH, CIERA_ST_BITMAP = 1, 2, 4, 8, 16
HEADER_BYTES = 64
CIERA_NOALLOC_SCRATCH_BYTES = 1 << 20  # the static scratch of ciera_encode_noalloc

# every symbol include/ciera.h declares
EXPORTS = ["ciera_plan", "ciera_plan_batch", "ciera_select", "ciera_shard", "ciera_encode_scratch_bytes", "ciera_encode",
           "ciera_encode_prepare", "ciera_encode_launch", "ciera_decode_scratch_bytes",
           "ciera_decode", "ciera_decode_prepare", "ciera_decode_launch", "ciera_cache_update",
           "ciera_hash_update", "ciera_set_sync_polls", "ciera_encode_noalloc", "ciera_decode_launch_bounded",
           "ciera_status_str", "ciera_abi_version", "ciera_last_error"]


class CieraError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        detail = f" [{_lib.ciera_last_error().decode()}]" if code == CIERA_ERR_DEVICE else ""
        super().__init__(f"{where}: {_lib.ciera_status_str(code).decode()} ({code}){detail}")


class Tensor(ctypes.Structure):
    _fields_ = [("rows", c_uint64), ("cols", c_uint64), ("dtype", c_uint32),
                ("block_size", c_uint32), ("world", c_uint32), ("flags", c_uint32)]

    def __init__(self, rows=0, cols=1, dtype=CIERA_BF16, block_size=512, world=1, flags=0):
        super().__init__(rows, cols, dtype, block_size, world, flags)


class CostModel(ctypes.Structure):
    _fields_ = [("link_bytes_per_us", c_uint64), ("hbm_bytes_per_us", c_uint64),
                ("fixed_ns", c_uint64), ("overlap_encode", c_uint32), ("reserved", c_uint32)]

    def __init__(self, link_bytes_per_us=8000, hbm_bytes_per_us=5_600_000, fixed_ns=5000,
                 overlap_encode=1):
        super().__init__(link_bytes_per_us, hbm_bytes_per_us, fixed_ns, overlap_encode, 0)


class Plan(ctypes.Structure):
    _fields_ = [("compress", c_uint32), ("reserved", c_uint32), ("raw_stream_bytes", c_uint64),
                ("max_stream_bytes", c_uint64), ("expected_stream_bytes", c_uint64),
                ("expected_changed", c_uint64), ("cache_bytes", c_uint64), ("gain_ns", c_int64)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


class EncodeItem(ctypes.Structure):
    _fields_ = [("t", Tensor), ("rank", c_uint32), ("compress", c_uint32), ("shard", c_void_p),
                ("cache_full", c_void_p), ("stream", c_void_p), ("stream_capacity", c_uint64)]


class DecodeItem(ctypes.Structure):
    _fields_ = [("t", Tensor), ("streams", c_void_p), ("slot_bytes", c_uint64),
                ("out_full", c_void_p), ("cache_full", c_void_p), ("rank_streams", c_void_p)]


class Batch(ctypes.Structure):
    """Host handle of a prepared batch (CIERA_BATCH_BYTES opaque bytes)."""
    _fields_ = [("opaque", c_uint64 * 512)]


def _hip_runtimes() -> set:
    """Paths of every HIP runtime library mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950) first")
    # torch ships its own HIP runtime under the same soname.  Loading torch first
    # makes libciera.so bind to that copy; loading libciera.so first would map a
    # second HIP/HSA runtime into the process, and one of them then finds no GPU.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    sig = {
        "ciera_plan": (c_int, [POINTER(Tensor), c_uint32, POINTER(CostModel), POINTER(Plan)]),
        "ciera_plan_batch": (c_int, [POINTER(Tensor), POINTER(c_uint32), c_uint32, POINTER(CostModel),
                                     POINTER(Plan)]),
        "ciera_select": (c_int, [POINTER(Plan), c_uint32, c_uint64, POINTER(c_uint32)]),
        "ciera_shard": (c_int, [POINTER(Tensor), c_uint32, POINTER(c_uint64), POINTER(c_uint64)]),
        "ciera_encode_scratch_bytes": (c_int, [POINTER(EncodeItem), c_uint32, POINTER(c_uint64)]),
        "ciera_encode": (c_int, [POINTER(EncodeItem), c_uint32, c_void_p, c_uint64, c_void_p]),
        "ciera_decode_scratch_bytes": (c_int, [POINTER(DecodeItem), c_uint32, POINTER(c_uint64)]),
        "ciera_decode": (c_int, [POINTER(DecodeItem), c_uint32, c_void_p, c_void_p, c_uint64, c_void_p]),
        "ciera_encode_prepare": (c_int, [POINTER(EncodeItem), c_uint32, c_void_p, c_uint64, POINTER(Batch),
                                         c_void_p]),
        "ciera_encode_launch": (c_int, [POINTER(Batch), c_void_p]),
        "ciera_decode_prepare": (c_int, [POINTER(DecodeItem), c_uint32, c_void_p, c_void_p, c_uint64,
                                         POINTER(Batch), c_void_p]),
        "ciera_decode_launch": (c_int, [POINTER(Batch), c_void_p]),
        "ciera_decode_launch_bounded": (c_int, [POINTER(Batch), c_uint32, c_void_p]),
        "ciera_cache_update": (c_int, [POINTER(Tensor), c_void_p, c_void_p, c_void_p]),
        "ciera_hash_update": (c_int, [POINTER(Tensor), c_uint32, c_void_p, c_void_p, c_void_p]),
        "ciera_set_sync_polls": (None, [c_uint32]),
        "ciera_encode_noalloc": (c_int, [POINTER(EncodeItem), c_uint32, c_void_p]),
        "ciera_status_str": (c_char_p, [c_int]),
        "ciera_abi_version": (c_uint32, []),
        "ciera_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()


def _check(code: int, where: str) -> None:
    if code != CIERA_OK:
        raise CieraError(code, where)


def _torch_dtype(ciera_dtype: int):
    import torch
    return {CIERA_BF16: torch.bfloat16, CIERA_FP32: torch.float32, CIERA_FP16: torch.float16}[ciera_dtype]


def _ptr(t, what: str = "buffer", dtype=None, numel: Optional[int] = None,
         min_numel: Optional[int] = None) -> Optional[int]:
    """Device address of a torch tensor (or an int address, or None).  The
    library reads and writes memory from that address on, so a torch tensor
    must be contiguous, of the element type and count the call implies (where
    it is given) and on a GPU; a strided view or a shard of another length
    would otherwise be read as the wrong memory (ValueError)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"{what}: not contiguous (shape {tuple(t.shape)}, stride {t.stride()})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what}: {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{what}: {t.numel()} elements, at least {min_numel} needed")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: on {t.device}, not on a GPU")
    return t.data_ptr()


def _u8(t, what: str, min_numel: int) -> Optional[int]:
    """A byte buffer (cache, stream, scratch, status) of at least min_numel bytes."""
    if t is None or isinstance(t, int):
        return t
    return _ptr(t, what, min_numel=-(-min_numel // t.element_size()))


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _items_array(cls, items: Sequence):
    arr = (cls * max(len(items), 1))()
    for i, it in enumerate(items):
        arr[i] = it
    return arr


# ------------------------------------------------------------------ host calls

def ciera_abi_version() -> int:
    return _lib.ciera_abi_version()


def ciera_status_str(code: int) -> str:
    return _lib.ciera_status_str(code).decode()


def ciera_plan(t: Tensor, change_ppm: int, cost: Optional[CostModel] = None) -> Plan:
    out = Plan()
    _check(_lib.ciera_plan(byref(t), change_ppm, byref(cost) if cost is not None else None,
                           byref(out)), "ciera_plan")
    return out


class PlanBatch:
    """Host arrays for ciera_plan_batch over a fixed list of tensors, built once
    so that a per-iteration plan of a whole layer is one library call."""

    def __init__(self, tensors: Sequence[Tensor], change_ppm, cost: Optional[CostModel] = None):
        n = len(tensors)
        self.count = n
        self.tensors = (Tensor * max(n, 1))(*tensors)
        ppm = [change_ppm] * n if isinstance(change_ppm, int) else list(change_ppm)
        if len(ppm) != n:
            raise ValueError(f"change_ppm: {len(ppm)} rates for {n} tensors")
        self.ppm = (c_uint32 * max(n, 1))(*ppm)
        self.cost = cost
        self.out = (Plan * max(n, 1))()

    def run(self):
        """Plans of every tensor (the array is reused by the next run)."""
        _check(_lib.ciera_plan_batch(self.tensors, self.ppm, self.count,
                                     byref(self.cost) if self.cost is not None else None, self.out),
               "ciera_plan_batch")
        return self.out


def ciera_plan_batch(tensors: Sequence[Tensor], change_ppm, cost: Optional[CostModel] = None) -> List[Plan]:
    """ciera_plan of every tensor in one call (change_ppm: one rate or one per tensor)."""
    b = PlanBatch(tensors, change_ppm, cost)
    return [Plan.from_buffer_copy(p) for p in b.run()[:b.count]]


def ciera_select(plans: Sequence[Plan], cache_budget_bytes: int) -> List[int]:
    """Benefit-driven selection: compress flag per plan under a cache budget."""
    arr = (Plan * max(len(plans), 1))()
    for i, p in enumerate(plans):
        arr[i] = p
    out = (c_uint32 * max(len(plans), 1))()
    _check(_lib.ciera_select(arr, len(plans), cache_budget_bytes, out), "ciera_select")
    return [int(out[i]) for i in range(len(plans))]


def ciera_shard(t: Tensor, rank: int) -> Tuple[int, int]:
    off, n = c_uint64(), c_uint64()
    _check(_lib.ciera_shard(byref(t), rank, byref(off), byref(n)), "ciera_shard")
    return off.value, n.value


def ciera_set_sync_polls(polls: int) -> None:
    """Bound on an encode tile's polls of a sibling's count before it counts
    that sibling's changes itself (0: the default)."""
    _lib.ciera_set_sync_polls(polls)


def ciera_encode_scratch_bytes(items: Sequence[EncodeItem]) -> int:
    b = c_uint64()
    _check(_lib.ciera_encode_scratch_bytes(_items_array(EncodeItem, items), len(items), byref(b)),
           "ciera_encode_scratch_bytes")
    return b.value


def ciera_decode_scratch_bytes(items: Sequence[DecodeItem]) -> int:
    b = c_uint64()
    _check(_lib.ciera_decode_scratch_bytes(_items_array(DecodeItem, items), len(items), byref(b)),
           "ciera_decode_scratch_bytes")
    return b.value


# ---------------------------------------------------------------- device calls

def encode_item(t: Tensor, rank: int, compress: int, shard, cache_full, stream_buf,
                capacity: Optional[int] = None) -> EncodeItem:
    cap = capacity if capacity is not None else stream_buf.numel() * stream_buf.element_size()
    off, n = ciera_shard(t, rank)
    state = (16 * (-(-n // t.block_size)) if compress == BLOCK else t.rows * t.cols)
    return EncodeItem(t, rank, int(compress),
                      _ptr(shard, "shard", None if isinstance(shard, int) else _torch_dtype(t.dtype), n),
                      _u8(cache_full, "hash cache" if compress == BLOCK else "cache", state),
                      _u8(stream_buf, "stream", 0), cap)


def decode_item(t: Tensor, streams, slot_bytes: int, out_full, cache_full, rank_streams=None) -> DecodeItem:
    """The W streams of t either as W slots of slot_bytes in `streams`, or,
    with streams None, as `rank_streams`: one buffer (or address) per rank,
    each of at least slot_bytes bytes.  The item keeps the host array of rank
    pointers alive."""
    N = t.rows * t.cols
    ranks = None
    if rank_streams is not None:
        if len(rank_streams) != t.world:
            raise ValueError(f"rank_streams: {len(rank_streams)} buffers, expected {t.world}")
        ranks = (c_void_p * t.world)(*[_u8(b, f"rank_streams[{r}]", slot_bytes) for r, b in enumerate(rank_streams)])
    item = DecodeItem(t, _u8(streams, "streams", slot_bytes * t.world),
                      slot_bytes,
                      _ptr(out_full, "out_full", None if out_full is None or isinstance(out_full, int)
                           else _torch_dtype(t.dtype), N),
                      _u8(cache_full, "cache", N),
                      None if ranks is None else ctypes.cast(ranks, c_void_p).value)
    item._ranks = ranks
    return item


def ciera_encode(items: Sequence[EncodeItem], scratch, scratch_bytes: Optional[int] = None,
                 stream=None) -> None:
    nbytes = scratch_bytes if scratch_bytes is not None else scratch.numel() * scratch.element_size()
    _check(_lib.ciera_encode(_items_array(EncodeItem, items), len(items), _ptr(scratch), nbytes,
                             _stream(stream)), "ciera_encode")


def ciera_encode_noalloc(items: Sequence[EncodeItem], stream=None) -> None:
    """ciera_encode with the library's static device scratch (no allocation)."""
    _check(_lib.ciera_encode_noalloc(_items_array(EncodeItem, items), len(items), _stream(stream)),
           "ciera_encode_noalloc")


def ciera_decode(items: Sequence[DecodeItem], status, scratch, scratch_bytes: Optional[int] = None,
                 stream=None) -> None:
    nbytes = scratch_bytes if scratch_bytes is not None else scratch.numel() * scratch.element_size()
    _check(_lib.ciera_decode(_items_array(DecodeItem, items), len(items), _ptr(status), _ptr(scratch),
                             nbytes, _stream(stream)), "ciera_decode")


def ciera_cache_update(t: Tensor, weights_full, cache_full, stream=None) -> None:
    N = t.rows * t.cols
    w = _ptr(weights_full, "weights_full",
             None if weights_full is None or isinstance(weights_full, int) else _torch_dtype(t.dtype), N)
    _check(_lib.ciera_cache_update(byref(t), w, _u8(cache_full, "cache", N), _stream(stream)),
           "ciera_cache_update")


def ciera_hash_update(t: Tensor, rank: int, shard, hash_cache, stream=None) -> None:
    off, n = ciera_shard(t, rank)
    x = _ptr(shard, "shard", None if shard is None or isinstance(shard, int) else _torch_dtype(t.dtype), n)
    _check(_lib.ciera_hash_update(byref(t), rank, x, _u8(hash_cache, "hash cache", 16 * (-(-n // t.block_size))),
                                  _stream(stream)), "ciera_hash_update")


def ciera_encode_prepare(items: Sequence[EncodeItem], scratch, scratch_bytes: Optional[int] = None,
                         stream=None) -> Batch:
    nbytes = scratch_bytes if scratch_bytes is not None else scratch.numel() * scratch.element_size()
    b = Batch()
    _check(_lib.ciera_encode_prepare(_items_array(EncodeItem, items), len(items), _ptr(scratch), nbytes,
                                     byref(b), _stream(stream)), "ciera_encode_prepare")
    return b


def ciera_encode_launch(batch: Batch, stream=None) -> None:
    _check(_lib.ciera_encode_launch(byref(batch), _stream(stream)), "ciera_encode_launch")


def ciera_decode_prepare(items: Sequence[DecodeItem], status, scratch, scratch_bytes: Optional[int] = None,
                         stream=None) -> Batch:
    nbytes = scratch_bytes if scratch_bytes is not None else scratch.numel() * scratch.element_size()
    b = Batch()
    _check(_lib.ciera_decode_prepare(_items_array(DecodeItem, items), len(items), _ptr(status), _ptr(scratch),
                                     nbytes, byref(b), _stream(stream)), "ciera_decode_prepare")
    return b


def ciera_decode_launch(batch: Batch, stream=None) -> None:
    _check(_lib.ciera_decode_launch(byref(batch), _stream(stream)), "ciera_decode_launch")


def ciera_decode_launch_bounded(batch: Batch, max_workgroups: int, stream=None) -> None:
    _check(_lib.ciera_decode_launch_bounded(byref(batch), max_workgroups, _stream(stream)),
           "ciera_decode_launch_bounded")
