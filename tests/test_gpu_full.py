"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (batched, prepared launches).

Every stream of every rank and tensor is compared byte for byte with the
oracle's (for the coded variant, whose oracle is pure Python, every header's
size and change count are checked against counts made here, and sampled
tensors byte for byte); the GPU's cache before each iteration is compared with
the oracle's; every output is checked on the GPU by properties that hold at
any size (decode(encode(x)) == x bit for bit, cache == exponent field of x, no
status bits); sampled tensors' rebuilt values and caches are compared with the
oracle's decode."""
import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import ciera_oracle as O

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lossless_weight_compression_amd.layer import LayerCodec  # noqa: E402
from tests.gpu_harness import Case, say, to_np  # noqa: E402

IV = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.float16: torch.int16}
ODT = {torch.bfloat16: O.BF16, torch.float32: O.FP32, torch.float16: O.FP16}


def exp_field_gpu(w: torch.Tensor) -> torch.Tensor:
    """Exponent byte of every value, computed on the GPU from the bit pattern
    (test-side property check, independent of the library)."""
    if w.dtype == torch.bfloat16:
        return ((w.reshape(-1).view(torch.int16).to(torch.int32) >> 7) & 0xFF).to(torch.uint8)
    if w.dtype == torch.float16:
        return ((w.reshape(-1).view(torch.int16).to(torch.int32) >> 10) & 0x1F).to(torch.uint8)
    return ((w.reshape(-1).view(torch.int32) >> 23) & 0xFF).to(torch.uint8)


def run_layer(specs, w_prev, w_next, dtype, world, ppm, codec=None, sample=(), seed_cache=True,
              expect_modes=None, coded=False):
    """Encode every rank (rank 0 prepared, the others one-shot), compare every
    stream with the oracle, decode with the prepared batch, check properties at
    full size and sampled tensors' decode against the oracle.  Returns the
    codec (cache carried) and a summary."""
    shapes = [(s.rows, s.cols) for s in specs]
    comp = [3] * len(specs) if coded else None  # coded patches for every tensor
    if codec is None:
        codec = LayerCodec(shapes, dtype, world, 512, "cuda", ppm, coded=[coded] * len(specs))
    else:
        codec.plans = [__import__("lossless_weight_compression_amd").ciera_plan(t, ppm) for t in codec.tensors]
    if seed_cache:
        codec.seed_cache(w_prev)
    torch.cuda.synchronize()
    for r in range(world):
        shards = []
        for i in range(len(specs)):
            off, n = codec.shard(i, r)
            shards.append(w_next[i].reshape(-1)[off:off + n])
        if r == 0:
            codec.prepare_encode(0, shards, compress=comp).launch()
        else:
            codec.encode(r, shards, compress=comp)
    torch.cuda.synchronize()
    # every stream against the oracle, tensor by tensor; the cache the encode
    # read (encode leaves it alone) against the oracle's cache of w_prev
    ocache, o_streams = {}, {}
    shift, em = {O.BF16: (7, 0xFF), O.FP32: (23, 0xFF), O.FP16: (10, 0x1F)}[ODT[dtype]]
    for i in range(len(specs)):
        s = specs[i]
        x = to_np(w_next[i])
        oc = O.cache_update(to_np(w_prev[i]), ODT[dtype])
        assert np.array_equal(codec.cache_view(i).cpu().numpy(), oc), f"cache before, tensor {i}"
        if i in sample:
            ocache[i] = oc
            o_streams[i] = []
        for r in range(world):
            off, n = O.shard(s.rows, s.cols, world, r)
            if not coded or i in sample:
                if coded:
                    st = O.encode_coded(x[off:off + n], oc[off:off + n], ODT[dtype], 512, True, off, r, world)
                else:
                    st = O.encode(x[off:off + n], oc[off:off + n], ODT[dtype], 512,
                                  bool(codec.plans[i].compress), off, r, world)
                got = codec.slot(i, r)[:st.size].cpu().numpy()
                assert np.array_equal(got, st), f"tensor {i} rank {r}: stream differs from the oracle"
                if i in sample:
                    o_streams[i].append(st)
            else:  # coded, not sampled: the header's size and change count
                hd = O.parse_header(codec.slot(i, r)[:64].cpu().numpy())
                changed = int(np.count_nonzero(((x[off:off + n] >> shift) & em) != oc[off:off + n]))
                assert hd["n"] == n and hd["n_changed"] == changed and hd["offset"] == off, \
                    f"tensor {i} rank {r}: header {hd}"
    status = codec.decode()
    torch.cuda.synchronize()
    assert status.item() == 0, f"decode status {status.item()}"
    # properties at full size
    for i in range(len(specs)):
        assert torch.equal(codec.out_view(i).view(IV[dtype]), w_next[i].reshape(-1).view(IV[dtype])), \
            f"tensor {i}: decode(encode(x)) != x"
        assert torch.equal(codec.cache_view(i), exp_field_gpu(w_next[i])), f"tensor {i}: cache != exponents"
    # sampled decode against the oracle
    for i in sample:
        s = specs[i]
        out, cache, st = O.decode(o_streams[i], s.rows, s.cols, ODT[dtype], 512, world, ocache[i], coded=coded)
        assert st == 0
        assert np.array_equal(to_np(codec.out_view(i)), out)
        assert np.array_equal(codec.cache_view(i).cpu().numpy(), cache)
    # headers: modes and sizes
    modes, total, raw = [], 0, 0
    for i in range(len(specs)):
        for r in range(world):
            h = codec.slot(i, r)[:64].cpu().numpy()
            hd = O.parse_header(h)
            modes.append(hd["mode"])
            total += hd["total_len"]
            raw += O.raw_len(hd["n"], ODT[dtype])
    if expect_modes is not None:
        expect_modes(np.array(modes).reshape(len(specs), world), codec)
    return codec, dict(ratio=raw / total, modes=modes)


def _layer(name, frac, clustered=False, device="cuda"):
    specs, cfg, world = W.config(name, frac=frac, clustered=clustered)
    win = W.layer_windows(specs, cfg)
    w0, w1 = [], []
    for i in range(len(specs)):
        a, b = W.weight_pair(specs, i, cfg, device=device, windows=win)
        w0.append(a)
        w1.append(b)
    return specs, cfg, world, w0, w1


EXPECTED_RATIO = {0.0: 2.0, 0.001: 1.989, 0.01: 1.904, 0.1: 1.333}


@pytest.mark.parametrize("clustered", [False, True])
@pytest.mark.parametrize("frac", [0.0, 0.001, 0.01, 0.1])
def test_olmoe_layer_bf16(frac, clustered):
    say(f"[gpu] OLMoE layer bf16 f={frac} clustered={clustered}")
    specs, cfg, world, w0, w1 = _layer("layer", frac, clustered)
    ppm = int(round(frac * 1e6))
    sample = (0, 97, 191)
    _, res = run_layer(specs, w0, w1, torch.bfloat16, world, ppm, sample=sample)
    say(f"[gpu]   compression ratio {res['ratio']:.4f}")
    # raw/compressed ~ 2 / (1 + 5f) either way (clustered shards with > ~20% changes go RAW)
    assert abs(res["ratio"] - EXPECTED_RATIO[frac]) < (0.01 if not clustered else 0.03)


# raw/streams with coded patches (a change costs about 16 bits at 1%)
EXPECTED_RATIO_CODED = {0.01: 1.956, 0.1: 1.780}


@pytest.mark.parametrize("frac,clustered,sample", [(0.01, False, (0, 97, 191)), (0.1, False, (0, 191)),
                                                   (0.01, True, (0, 97, 191))])
def test_olmoe_layer_bf16_coded(frac, clustered, sample):
    """The full layer with every tensor's changes range-ANS coded (stream mode
    3), in the prepared launch bench.py --variant coded times."""
    say(f"[gpu] OLMoE layer bf16 coded f={frac} clustered={clustered}")
    specs, cfg, world, w0, w1 = _layer("layer", frac, clustered)
    ppm = int(round(frac * 1e6))

    def modes_all_coded(m, codec):
        assert (m == O.MODE_CODED).all()

    _, res = run_layer(specs, w0, w1, torch.bfloat16, world, ppm, sample=sample, coded=True,
                       expect_modes=modes_all_coded)
    say(f"[gpu]   compression ratio {res['ratio']:.4f}")
    if not clustered:
        assert abs(res["ratio"] - EXPECTED_RATIO_CODED[frac]) < 0.01


@pytest.mark.parametrize("frac", [0.0, 0.01, 0.1])
def test_olmoe_layer_fp16(frac):
    """The 64-expert layer in fp16: 11-bit sign|mantissa stream, raw/compressed
    ~ 2 / (1.375 + 5f) (still below 2 at 10%; the break-even is 12.5%)."""
    say(f"[gpu] OLMoE layer fp16 f={frac}")
    specs, cfg, world, w0, w1 = _layer("layer_fp16", frac)
    ppm = int(round(frac * 1e6))
    _, res = run_layer(specs, w0, w1, torch.float16, world, ppm, sample=(0, 97, 191))
    say(f"[gpu]   compression ratio {res['ratio']:.4f}")
    want = 2.0 / min(2.0, 1.375 + 5 * frac)
    assert abs(res["ratio"] - want) < 0.02


def test_olmoe_layer_fp32_warmup_and_schedule():
    """fp32 master weights: 30% warmup makes every tensor RAW by plan; then
    30% -> 5% -> 0.5% over three iterations with the cache carried and the
    plan re-run each iteration."""
    specs = W.olmoe_layer_specs()
    world = 16
    cfg = W.PairConfig("fp32-sched", dtype=torch.float32)
    w = [W.base_weights(s, W.tensor_seed("fp32-sched", "base", i), torch.float32, "cuda")
         for i, s in enumerate(specs)]
    codec = None
    for it, frac in enumerate((0.30, 0.05, 0.005)):
        say(f"[gpu] fp32 layer iteration {it} f={frac}")
        nxt = []
        for i, s in enumerate(specs):
            m = W.mask_uniform(s.numel, frac, W.tensor_seed("fp32-sched", "mask", i, it), "cuda")
            nxt.append(W.perturb_exact(w[i], m, W.tensor_seed("fp32-sched", "next", i, it)))
        ppm = int(round(frac * 1e6))

        def modes_ok(modes, c, frac=frac):
            plans = np.array([p.compress for p in c.plans])
            if frac >= 0.3:
                assert plans.sum() == 0 and (modes == O.MODE_RAW).all()
            else:
                assert plans.all() and (modes == O.MODE_COMPRESSED).all()
        codec, res = run_layer(specs, w, nxt, torch.float32, world, ppm, codec=codec,
                               sample=(0, 100), seed_cache=(it == 0), expect_modes=modes_ok)
        say(f"[gpu]   compression ratio {res['ratio']:.4f}")
        w = nxt


def test_olmoe_layer_fp32_forced_compress_falls_back_raw():
    """Plan overridden to compress at 30% change: every stream must come out RAW
    through the fallback rewrite, bit-exact."""
    specs = W.olmoe_expert_specs()
    cfg = W.PairConfig("fp32-force", dtype=torch.float32, frac=0.30)
    w0, w1 = [], []
    for i in range(len(specs)):
        a, b = W.weight_pair(specs, i, cfg, device="cuda")
        w0.append(a)
        w1.append(b)
    codec = LayerCodec([(s.rows, s.cols) for s in specs], torch.float32, 16, 512, "cuda", 10000)
    assert all(p.compress for p in codec.plans)

    def all_raw(modes, c):
        assert (modes == O.MODE_RAW).all()
    run_layer(specs, w0, w1, torch.float32, 16, 10000, codec=codec, sample=(0, 2), expect_modes=all_raw)


def test_fine_grained_layer_with_specials():
    """256 experts x (7168x2048, 7168x2048, 2048x7168) + router 7168x256 + two
    RMSNorm vectors of 7168 (11.28 G bf16 values), 1% changes, 1e-4 specials:
    the plan keeps the RMSNorm shards RAW and compresses experts and router."""
    say("[gpu] fine-grained layer: generating 2 x 22.6 GB")
    specs, cfg, world, w0, w1 = _layer("fine", 0.01)
    n_t = len(specs)

    def modes_ok(modes, c):
        plans = [p.compress for p in c.plans]
        for i, s in enumerate(specs):
            if s.name.startswith("norm"):
                assert plans[i] == 0 and (modes[i] == O.MODE_RAW).all()
            else:
                assert plans[i] == 1 and (modes[i] == O.MODE_COMPRESSED).all()
    say("[gpu] fine-grained layer: encode 16 ranks, decode")
    _, res = run_layer(specs, w0, w1, torch.bfloat16, world, 10000,
                       sample=(0, n_t - 3, n_t - 2, n_t - 1), expect_modes=modes_ok)
    say(f"[gpu]   compression ratio {res['ratio']:.4f}")


def test_prepared_batch_rejects_foreign_scratch():
    """A prepared batch whose scratch was taken over by another batch writes
    nothing (its kernels see the other batch id and exit)."""
    import lossless_weight_compression_amd as L
    specs = W.olmoe_expert_specs()
    cfg = W.PairConfig("foreign", frac=0.01)
    w0, w1 = [], []
    for i in range(len(specs)):
        a, b = W.weight_pair(specs, i, cfg, device="cuda")
        w0.append(a)
        w1.append(b)
    codec = LayerCodec([(s.rows, s.cols) for s in specs], torch.bfloat16, 16, 512, "cuda", 10000)
    codec.seed_cache(w0)
    shards = [w1[i].reshape(-1)[:codec.shard(i, 0)[1]] for i in range(3)]
    items = codec.encode_items(0, shards)
    scratch = torch.empty(L.ciera_encode_scratch_bytes(items), dtype=torch.uint8, device="cuda")
    a = L.ciera_encode_prepare(items, scratch)
    b = L.ciera_encode_prepare(items, scratch)   # takes the scratch over
    codec.streams.zero_()
    L.ciera_encode_launch(a)
    torch.cuda.synchronize()
    assert int(codec.streams.count_nonzero()) == 0
    L.ciera_encode_launch(b)
    torch.cuda.synchronize()
    assert int(codec.streams.count_nonzero()) > 0


def test_layer_under_cache_budget():
    """ciera_select inside LayerCodec: with a cache budget of two expert
    tensors, the norm (no gain), the router and one expert go RAW, the two
    other experts COMPRESSED; the round trip stays bit-exact and the streams
    equal the oracle's for those decisions."""
    shapes = [(7168, 1), (7168, 256), (2048, 1024), (2048, 1024), (1024, 2048)]
    say(f"[gpu] cache budget {shapes}")
    budget = 2 * 2048 * 1024
    codec = LayerCodec(shapes, torch.bfloat16, 16, change_ppm=10_000, cache_budget=budget)
    want = O.select([p.gain_ns for p in codec.plans], [p.cache_bytes for p in codec.plans], budget)
    got = [p.compress for p in codec.plans]
    assert got == want and sum(got) == 2, got
    w0, w1 = [], []
    for i, (r, c) in enumerate(shapes):
        spec = W.TensorSpec(f"t{i}", r, c)
        a = W.base_weights(spec, W.tensor_seed("budget", i), torch.bfloat16)
        m = W.mask_uniform(r * c, 0.01, W.tensor_seed("budget-m", i))
        w0.append(a)
        w1.append(W.perturb_exact(a, m, W.tensor_seed("budget-p", i)))
    case = Case(shapes, torch.bfloat16, 16)
    res = case.run(w0, w1, compress=got)
    assert res["status"] == 0 and res["ostatus"] == 0
    modes = [int(O.parse_header(case.codec.slot(i, 0).cpu().numpy())["mode"]) for i in range(len(shapes))]
    assert modes == [O.MODE_COMPRESSED if g else O.MODE_RAW for g in got]

