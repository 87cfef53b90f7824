"""The codec under HIP graph capture.  A step -- clear the status word, encode
one rank's shards (the prepared encode, or the allocation-free one), decode
every tensor from its W streams -- captured into one graph and replayed
several times, with the program's own eager work between the replays (other
encodes through the same static scratch, unrelated kernels, resets of the
cache and of the buffers the step writes).  Every replay's streams, rebuilt
values, caches and status must equal those of the same calls run eagerly.
The captured calls enqueue kernels only (no memset or copy nodes: the status
word is cleared by a fill kernel, the allocation-free encode passes its
descriptors as kernel arguments)."""
import numpy as np
import pytest
import torch

from gen import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import lossless_weight_compression_amd as L  # noqa: E402
from lossless_weight_compression_amd.layer import LayerCodec  # noqa: E402
from tests.gpu_harness import say  # noqa: E402

SHAPES = [(512, 768), (96, 4096), (7, 5), (64, 3000), (2048, 1024)]
WORLD = 4


def _setup(dtype, tag):
    codec = LayerCodec(SHAPES, dtype, WORLD, 512, "cuda", 10_000)
    w0, w1 = [], []
    for i, (r, c) in enumerate(SHAPES):
        s = W.TensorSpec(f"{tag}{i}", r, c)
        a = W.base_weights(s, W.tensor_seed(tag, i), dtype).cuda()
        m = W.mask_uniform(s.numel, 0.02, W.tensor_seed(tag + "-m", i)).cuda()
        w0.append(a)
        w1.append(W.perturb_exact(a, m, W.tensor_seed(tag + "-p", i)))
    codec.seed_cache(w0)
    shards = {}
    for r in range(WORLD):
        shards[r] = []
        for i in range(len(SHAPES)):
            off, n = codec.shard(i, r)
            shards[r].append(w1[i].reshape(-1)[off:off + n].clone())
    for r in range(1, WORLD):  # the other ranks' streams stay in their slots
        codec.encode(r, shards[r])
    torch.cuda.synchronize()
    return codec, w1, shards


def _rank0_slots(codec):
    return [codec.slot(i, 0) for i in range(len(SHAPES))]


def _reset(codec, cache0):
    """Undo what a step writes: the cache back to the seed, rank 0's slots,
    the rebuilt values and the status word overwritten."""
    codec.cache.copy_(cache0)
    for s in _rank0_slots(codec):
        s.fill_(0xA5)
    codec.out.fill_(0x5A)
    codec.status.fill_(7)


def _state(codec):
    torch.cuda.synchronize()
    return codec.streams.clone(), codec.out.clone(), codec.cache.clone(), int(codec.status.item())


def _check(codec, ref, got, w1, rep):
    streams, out, cache, status = got
    r_streams, r_out, r_cache, r_status = ref
    assert status == r_status == 0, (rep, status, r_status)
    for i in range(len(SHAPES)):
        a0 = codec.stream_off[i]
        for r in range(WORLD):
            lo = a0 + r * codec.slot_bytes[i]
            want = r_streams[lo:lo + codec.slot_bytes[i]].cpu().numpy()
            total = int(want[32:40].view(np.uint64)[0])
            got_s = streams[lo:lo + total].cpu().numpy()
            assert np.array_equal(got_s, want[:total]), (rep, i, r)
        n = codec.numel[i]
        o = codec.out_off[i]
        e = codec.e
        assert torch.equal(out[o:o + n * e], r_out[o:o + n * e]), (rep, i)
        assert torch.equal(out[o:o + n * e].view(codec.dtype), w1[i].reshape(-1)), (rep, i)
        c = codec.cache_off[i]
        assert torch.equal(cache[c:c + n], r_cache[c:c + n]), (rep, i)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("noalloc", [False, True])
def test_captured_step_replays_like_eager_calls(dtype, noalloc):
    say(f"[gpu] graph capture {dtype} noalloc={noalloc}")
    codec, w1, shards = _setup(dtype, f"graph-{noalloc}")
    cache0 = codec.cache.clone()
    items0 = codec.encode_items(0, shards[0])
    prepared = codec.prepare_encode(0, shards[0])

    def step():
        codec.status.zero_()
        if noalloc:
            L.ciera_encode_noalloc(items0)
        else:
            prepared.launch()
        codec.decode(zero_status=False)

    # eager reference (this also prepares the decode batch and, for the
    # allocation-free encode, looks up the static scratch, outside the capture)
    _reset(codec, cache0)
    step()
    ref = _state(codec)
    _check(codec, ref, ref, w1, "eager")

    _reset(codec, cache0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    # an unrelated encode through the same static scratch, of a smaller batch
    other = LayerCodec(SHAPES[:2], dtype, WORLD, 512, "cuda", 10_000)
    other.seed_cache(w1[:2])
    o_items = other.encode_items(1, [shards[1][0], shards[1][1]])
    a = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        _reset(codec, cache0)
        if rep % 2:
            L.ciera_encode_noalloc(o_items)
        b = a @ a  # other eager work between replays
        g.replay()
        got = _state(codec)
        _check(codec, ref, got, w1, rep)
        assert torch.isfinite(b).all()
