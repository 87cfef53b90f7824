"""The codec on a side stream beside compute [CIERA 3.3, Figure 7: hash and
compress on their own stream, overlapped with communication and compute]:
encode of every rank and the decode run on a second HIP stream (default
priority) while bf16 GEMMs run on the first.  Streams, rebuilt values and
caches must equal the oracle's byte for byte, and the GEMM's result must equal
the same GEMM run alone."""
import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import ciera_oracle as O

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lossless_weight_compression_amd.layer import LayerCodec  # noqa: E402
from tests.gpu_harness import DT, IV, say, to_np  # noqa: E402


@pytest.mark.parametrize("dtype,frac", [(torch.bfloat16, 0.01), (torch.float32, 0.005), (torch.bfloat16, 0.3)])
def test_codec_on_a_side_stream_beside_a_gemm(dtype, frac):
    say(f"[gpu] overlap: {dtype} f={frac} codec on a side stream, GEMMs on the main one")
    specs = W.olmoe_expert_specs() + [W.TensorSpec("router", 7168, 256)]
    world = 16
    cfg = W.PairConfig(f"overlap-{frac}", dtype=dtype, frac=frac)
    w0, w1 = [], []
    for i in range(len(specs)):
        a, b = W.weight_pair(specs, i, cfg, device="cuda")
        w0.append(a)
        w1.append(b)
    shapes = [(s.rows, s.cols) for s in specs]
    codec = LayerCodec(shapes, dtype, world, 512, "cuda", int(frac * 1e6))
    shards = []
    for r in range(world):
        row = []
        for i in range(len(specs)):
            off, n = codec.shard(i, r)
            row.append(w1[i].reshape(-1)[off:off + n].clone())
        shards.append(row)
    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn(4096, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(8192, 4096, device="cuda", dtype=torch.bfloat16, generator=g)
    alone = torch.mm(a, b)
    c = torch.empty_like(alone)
    torch.cuda.synchronize()

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    start = torch.cuda.Event()
    start.record(main)
    side.wait_event(start)
    for _ in range(4):          # compute on the main stream ...
        torch.mm(a, b, out=c)
    codec.seed_cache(w0, stream=side)  # ... the whole codec on the side stream meanwhile
    for r in range(world):
        codec.encode(r, shards[r], stream=side)
    status = codec.decode(stream=side)
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    torch.cuda.synchronize()

    assert torch.equal(c, alone), "the GEMM beside the codec differs from the GEMM alone"
    assert int(status.item()) == 0
    _against_oracle(codec, specs, w0, w1, dtype, world)


def _against_oracle(codec, specs, w0, w1, dtype, world):
    """Every stream, rebuilt value and cache of the codec against the oracle."""
    for i, s in enumerate(specs):
        x0, x1 = to_np(w0[i]), to_np(w1[i])
        cache = O.cache_update(x0, DT[dtype])
        streams = []
        for r in range(world):
            off, n = O.shard(s.rows, s.cols, world, r)
            st = O.encode(x1[off:off + n], cache[off:off + n], DT[dtype], 512, bool(codec.plans[i].compress),
                          off, r, world)
            got = codec.slot(i, r)[:st.size].cpu().numpy()
            assert np.array_equal(got, st), f"tensor {i} rank {r}: stream differs from the oracle"
            streams.append(st)
        out, new_cache, ost = O.decode(streams, s.rows, s.cols, DT[dtype], 512, world, cache)
        assert ost == 0
        assert np.array_equal(to_np(codec.out_view(i)), out), f"tensor {i}: values differ"
        assert np.array_equal(codec.cache_view(i).cpu().numpy(), new_cache), f"tensor {i}: caches differ"
        assert torch.equal(codec.out_view(i).view(IV[dtype]), w1[i].reshape(-1).view(IV[dtype]))


@pytest.mark.parametrize("max_wg", [1, 7, 300])
def test_bounded_decode_grid(max_wg):
    """ciera_decode_launch_bounded: the decode from a grid of max_wg workgroups,
    each decoding tiles in turn, gives the oracle's values, caches and status;
    a corrupt stream is reported as by the unbounded decode."""
    say(f"[gpu] bounded decode grid {max_wg}")
    specs = W.olmoe_expert_specs() + [W.TensorSpec("odd", 333, 77)]
    world, dtype = 16, torch.bfloat16
    cfg = W.PairConfig("bounded", dtype=dtype, frac=0.01)
    w0, w1 = [], []
    for i in range(len(specs)):
        a, b = W.weight_pair(specs, i, cfg, device="cuda")
        w0.append(a)
        w1.append(b)
    codec = LayerCodec([(s.rows, s.cols) for s in specs], dtype, world, 512, "cuda", 10_000)
    codec.seed_cache(w0)
    for r in range(world):
        sh = []
        for i in range(len(specs)):
            off, n = codec.shard(i, r)
            sh.append(w1[i].reshape(-1)[off:off + n].clone())
        codec.encode(r, sh)
    status = codec.decode(max_workgroups=max_wg)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    _against_oracle(codec, specs, w0, w1, dtype, world)
    # a record index out of order in rank 5's stream of tensor 1: the same status bits
    codec.seed_cache(w0)
    slot = codec.slot(1, 5)
    n = codec.shard(1, 5)[1]
    pb = 64 + n + O.bitmap_bytes(n, 512)
    slot[pb:pb + 4] = slot[pb + 5:pb + 9].clone()
    st_b = int(codec.decode(max_workgroups=max_wg).item())
    codec.seed_cache(w0)
    st_u = int(codec.decode().item())
    torch.cuda.synchronize()
    assert st_b == st_u and st_u & O.ST_PATCH, (st_b, st_u)
