"""Decode from per-rank stream buffers (`rank_streams` of a decode item): the W
streams of a tensor in W device buffers of their own, as a receiver that does
not gather into one buffer holds them [CIERA 3.1; Algorithm 1 receiver].  The
rebuilt values, the caches and the status must equal those of the slot layout
and the oracle, for every stream mode, in batches that mix both layouts, and
through the bounded-grid launch."""
import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import ciera_oracle as O

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lossless_weight_compression_amd import _binding as B  # noqa: E402
from lossless_weight_compression_amd.layer import LayerCodec  # noqa: E402
from tests.gpu_harness import DT, say, to_np  # noqa: E402
from tests.test_gpu_coded import _pair  # noqa: E402

# (rows, cols, mode) per tensor: element patches, a plan-RAW stream, the
# block-hash variant, coded patches; shards from one value to several tiles
LAYER = [(512, 768, B.COMPRESSED), (96, 4096, B.CODED), (7, 5, B.COMPRESSED), (64, 3000, B.BLOCK),
         (33, 1000, B.RAW), (2048, 1024, B.COMPRESSED)]


def _encode(shapes, modes, dtype, world, block, frac, seed):
    """A codec holding every rank's stream of w1 against the w0 cache in its
    slots (each compared with the oracle by the other GPU tests)."""
    coded = [m == B.CODED for m in modes]
    codec = LayerCodec(shapes, dtype, world, block, "cuda", 10_000, coded=coded)
    pairs = [_pair(r, c, dtype, frac, (seed, i), steps=(1, -1, 3)) for i, (r, c) in enumerate(shapes)]
    w0 = [p[0] for p in pairs]
    w1 = [p[1] for p in pairs]
    d0 = [x.to("cuda").contiguous() for x in w0]
    d1 = [x.to("cuda").contiguous() for x in w1]
    codec.seed_cache(d0)

    def shards(ws, r):
        out = []
        for i in range(len(shapes)):
            off, n = codec.shard(i, r)
            out.append(ws[i].reshape(-1)[off:off + n].clone())
        return out

    for r in range(world):
        codec.seed_hashes(r, shards(d0, r))
    for r in range(world):
        codec.encode(r, shards(d1, r), compress=modes)
    torch.cuda.synchronize()
    return codec, w0, w1


def _rank_buffers(codec, i, rng, keep):
    """Rank r's slot copied to a buffer of its own, at a random 16-byte aligned
    place inside a larger allocation of filler bytes, allocated in a random rank
    order: the buffers are neither contiguous nor in rank order."""
    sb = codec.slot_bytes[i]
    bufs = [None] * codec.world
    for r in rng.permutation(codec.world):
        pad = 16 * int(rng.integers(0, 9))
        big = torch.full((pad + sb + 16 * int(rng.integers(0, 4)),), 0xA5, dtype=torch.uint8, device="cuda")
        big[pad:pad + sb] = codec.slot(i, r)
        bufs[int(r)] = big[pad:pad + sb]
        keep.append(big)
    return bufs


def _decode(codec, w0, use_ranks, rng, bounded=None, edit=None):
    """Decode every tensor of the codec's slots into fresh values and a cache
    seeded from w0; tensor i from per-rank buffers when use_ranks[i].  `edit`
    (i, r, offset, bytes) is applied to the copy that is decoded.  Returns
    (status, values, caches)."""
    keep, items, outs, caches = [], [], [], []
    for i, t in enumerate(codec.tensors):
        n = codec.numel[i]
        out = torch.empty(n, dtype=codec.dtype, device="cuda")
        cache = torch.from_numpy(O.cache_update(to_np(w0[i]), DT[codec.dtype])).to("cuda")
        if use_ranks[i]:
            bufs = _rank_buffers(codec, i, rng, keep)
            if edit is not None and edit[0] == i:
                _, r, o, b = edit
                bufs[r][o:o + len(b)] = torch.tensor(list(b), dtype=torch.uint8, device="cuda")
            items.append(B.decode_item(t, None, codec.slot_bytes[i], out, cache, rank_streams=bufs))
        else:
            sl = torch.empty(codec.slot_bytes[i] * codec.world, dtype=torch.uint8, device="cuda")
            for r in range(codec.world):
                sl[r * codec.slot_bytes[i]:(r + 1) * codec.slot_bytes[i]] = codec.slot(i, r)
            if edit is not None and edit[0] == i:
                _, r, o, b = edit
                a = r * codec.slot_bytes[i] + o
                sl[a:a + len(b)] = torch.tensor(list(b), dtype=torch.uint8, device="cuda")
            keep.append(sl)
            items.append(B.decode_item(t, sl, codec.slot_bytes[i], out, cache))
        outs.append(out)
        caches.append(cache)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(max(B.ciera_decode_scratch_bytes(items), 256), dtype=torch.uint8, device="cuda")
    if bounded is None:
        B.ciera_decode(items, status, scratch)
    else:
        batch = B.ciera_decode_prepare(items, status, scratch)
        B.ciera_decode_launch_bounded(batch, bounded)
    torch.cuda.synchronize()
    del keep
    return int(status.item()), outs, caches


@pytest.mark.parametrize("dtype,world,block", [(torch.bfloat16, 4, 512), (torch.float32, 3, 1024),
                                               (torch.float16, 16, 64)])
def test_every_mode_from_rank_buffers(dtype, world, block):
    say(f"[gpu] rank stream buffers {dtype} W={world} B={block}")
    shapes = [(r, c) for r, c, _ in LAYER]
    modes = [m for _, _, m in LAYER]
    codec, w0, w1 = _encode(shapes, modes, dtype, world, block, 0.02, 1)
    rng = np.random.default_rng(11)
    for use in ([True] * len(shapes), [i % 2 == 0 for i in range(len(shapes))]):
        st, outs, caches = _decode(codec, w0, use, rng)
        assert st == 0, (use, st)
        for i in range(len(shapes)):
            x1 = to_np(w1[i])
            assert np.array_equal(to_np(outs[i]), x1), (use, i)
            assert np.array_equal(caches[i].cpu().numpy(), O.cache_update(x1, DT[dtype])), (use, i)


def test_rank_buffers_through_the_bounded_grid():
    say("[gpu] rank stream buffers, bounded grid")
    shapes = [(512, 768), (2048, 1024), (7, 5)]
    modes = [B.COMPRESSED, B.COMPRESSED, B.RAW]
    codec, w0, w1 = _encode(shapes, modes, torch.bfloat16, 8, 512, 0.01, 2)
    rng = np.random.default_rng(12)
    for grid in (1, 7, 64):
        st, outs, caches = _decode(codec, w0, [True, False, True], rng, bounded=grid)
        assert st == 0, grid
        for i in range(len(shapes)):
            x1 = to_np(w1[i])
            assert np.array_equal(to_np(outs[i]), x1), (grid, i)
            assert np.array_equal(caches[i].cpu().numpy(), O.cache_update(x1, O.BF16)), (grid, i)


def test_rank_buffer_corruption_gives_the_slot_layouts_status():
    """The same byte edits in one rank's buffer and in that rank's slot give the
    same status (and the oracle's), for a record index past the shard, a header
    field and a coded chunk-table entry."""
    say("[gpu] rank stream buffers, corrupt streams")
    shapes = [(512, 768), (96, 4096)]
    modes = [B.COMPRESSED, B.CODED]
    world, block = 4, 512
    codec, w0, w1 = _encode(shapes, modes, torch.bfloat16, world, block, 0.02, 3)
    s0 = codec.slot(0, 2).cpu().numpy()
    h0 = O.parse_header(s0)
    n0 = int(h0["n"])
    pb = 64 + n0 + O.bitmap_bytes(n0, block)
    s1 = codec.slot(1, 1).cpu().numpy()
    h1 = O.parse_header(s1)
    assert h0["mode"] == O.MODE_COMPRESSED and h1["mode"] == O.MODE_CODED
    n1 = int(h1["n"])
    tpos = (64 + n1 + O.bitmap_bytes(n1, block) + 3) // 4 * 4
    edits = [(0, 2, pb + 5 * (int(h0["n_changed"]) - 1), (n0 + 3).to_bytes(4, "little")),   # index >= n
             (0, 2, 48, (3).to_bytes(4, "little")),                                        # rank field
             (1, 1, tpos, (1 << 20).to_bytes(4, "little"))]                                 # chunk table
    rng = np.random.default_rng(13)
    for e in edits:
        i, r, o, b = e
        st_slots, _, _ = _decode(codec, w0, [False, False], rng, edit=e)
        st_ranks, _, _ = _decode(codec, w0, [True, True], rng, edit=e)
        rows, cols = shapes[i]
        o_slots = []
        for rr in range(world):
            s = codec.slot(i, rr).cpu().numpy().copy()
            if rr == r:
                s[o:o + len(b)] = np.frombuffer(bytes(b), dtype=np.uint8)
            o_slots.append(s)
        cache0 = O.cache_update(to_np(w0[i]), O.BF16)
        _, _, ost = O.decode(o_slots, rows, cols, O.BF16, block, world, cache0, coded=modes[i] == B.CODED)
        assert ost != 0 and st_ranks == st_slots, (e[:3], st_ranks, st_slots, ost)
        if not ost & O.ST_PATCH:
            assert st_ranks == ost, (e[:3], st_ranks, ost)
        else:  # bitmap verdict unspecified alongside a patch error
            assert st_ranks & ~O.ST_BITMAP == ost & ~O.ST_BITMAP, (e[:3], st_ranks, ost)
