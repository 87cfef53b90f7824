"""GPU parity: the HIP path (through the C ABI) against the oracle, byte for byte.

Streams (header, sign|mantissa bytes, bitmap, patches), rebuilt values, caches
and decode status must be identical -- integer work, zero tolerance."""
import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import ciera_oracle as O

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these; be explicit anyway
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_harness import Case, say, to_np  # noqa: E402


def _pairs(specs, cfg, device="cpu"):
    win = W.layer_windows(specs, cfg)
    w0, w1 = [], []
    for i in range(len(specs)):
        a, b = W.weight_pair(specs, i, cfg, device=device, windows=win)
        w0.append(a)
        w1.append(b)
    return w0, w1


@pytest.mark.parametrize("name", ["tiny", "tiny2pct", "expert"])
def test_named_configs(name):
    specs, cfg, world = W.config(name)
    say(f"[gpu] config {name}: {[(s.rows, s.cols) for s in specs]} W={world}")
    w0, w1 = _pairs(specs, cfg)
    case = Case([(s.rows, s.cols) for s in specs], cfg.dtype, world)
    res = case.run(w0, w1)
    assert res["status"] == 0 and res["ostatus"] == 0
    rate = np.mean([np.mean(O.exponent_field(to_np(a), O.BF16) != O.exponent_field(to_np(b), O.BF16))
                    for a, b in zip(w0, w1)])
    say(f"[gpu] config {name}: exponent change rate {rate:.5%}")


EDGE = [
    # rows, cols, world, B, dtype, frac
    (1, 1, 1, 512, torch.bfloat16, 0.5),
    (17, 1, 16, 64, torch.bfloat16, 0.3),
    (3, 5, 8, 512, torch.bfloat16, 0.2),        # ranks 3..7 hold no rows
    (10, 3, 4, 64, torch.bfloat16, 0.1),        # shard offsets not 16-aligned
    (10, 3, 4, 64, torch.float32, 0.1),
    (33, 7, 2, 128, torch.float32, 0.05),
    (1, 4097, 1, 512, torch.bfloat16, 0.01),    # one value past a tile
    (2, 8193, 1, 64, torch.bfloat16, 0.002),
    (4101, 3, 3, 256, torch.bfloat16, 0.01),
    (64, 1000, 4, 1024, torch.bfloat16, 0.01),  # two 4096-value sub-tiles per tile
    (64, 1000, 4, 2048, torch.float32, 0.01),
    (96, 4096, 2, 4096, torch.bfloat16, 0.001),
    (96, 4096, 2, 4096, torch.float32, 0.0),
    (1000, 1000, 16, 512, torch.bfloat16, 0.0),
    (1000, 1000, 16, 512, torch.float32, 0.003),
    (7168, 1, 16, 512, torch.bfloat16, 0.01),   # an RMSNorm vector
    # fp16: 22-byte sign|mantissa chunks start mid-word at odd chunks; partial
    # chunks at every shard end that is not a multiple of 16 values
    (1, 1, 1, 512, torch.float16, 0.5),
    (17, 1, 16, 64, torch.float16, 0.3),
    (10, 3, 4, 64, torch.float16, 0.1),
    (33, 7, 2, 128, torch.float16, 0.05),
    (1, 4097, 1, 512, torch.float16, 0.01),
    (2, 8193, 1, 64, torch.float16, 0.002),
    (64, 1000, 4, 1024, torch.float16, 0.01),
    (1000, 1000, 16, 512, torch.float16, 0.003),
    (96, 4096, 2, 4096, torch.float16, 0.0),
]


@pytest.mark.parametrize("rows,cols,world,B,dtype,frac", EDGE)
def test_edge_shapes(rows, cols, world, B, dtype, frac):
    say(f"[gpu] edge {rows}x{cols} W={world} B={B} {dtype} f={frac}")
    spec = [W.TensorSpec("e", rows, cols)]
    w0 = [W.base_weights(spec[0], W.tensor_seed("edge", rows, cols, B), dtype)]
    mask = W.mask_uniform(rows * cols, frac, W.tensor_seed("edge-m", rows, cols, B))
    w1 = [W.perturb_exact(w0[0], mask, W.tensor_seed("edge-p", rows, cols, B))]
    for compress in ([1], [0]):
        case = Case([(rows, cols)], dtype, world, B)
        res = case.run(w0, w1, compress=compress)
        assert res["status"] == 0 and res["ostatus"] == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("frac", [0.0, 0.005, 0.19, 0.3, 1.0])
def test_change_rates_and_raw_fallback(dtype, frac):
    """Forced compress=1 at every rate: high rates must come out RAW through the
    fallback rewrite, low rates COMPRESSED."""
    say(f"[gpu] rates {dtype} f={frac}")
    specs = [W.TensorSpec("a", 256, 512), W.TensorSpec("b", 128, 1024), W.TensorSpec("c", 64, 333)]
    w0, w1 = [], []
    for i, s in enumerate(specs):
        a = W.base_weights(s, W.tensor_seed("rates", i), dtype)
        m = W.mask_uniform(s.numel, frac, W.tensor_seed("rates-m", i, frac))
        w0.append(a)
        w1.append(W.perturb_exact(a, m, W.tensor_seed("rates-p", i, frac)))
    case = Case([(s.rows, s.cols) for s in specs], dtype, 4)
    res = case.run(w0, w1, compress=[1, 1, 1])
    assert res["status"] == 0 and res["ostatus"] == 0
    modes = {int(O.parse_header(case.codec.slot(i, r).cpu().numpy())["mode"])
             for i in range(3) for r in range(4)}
    if frac >= 0.3:
        assert modes == {O.MODE_RAW}
    if frac <= 0.005:
        assert modes == {O.MODE_COMPRESSED}


# RAW fallback of shards of several encode tiles whose last tile is partial:
# the tiles store their sign|mantissa records before the item's total is
# known, and a RAW stream is then rewritten by the tiles that own its bytes.
# Tiles of 8192, 16384 and 32768 values (B 512, 2048, 4096); lengths that end
# mid-chunk (fp16: inside an 11-bit value's bytes); change rates from all RAW
# to around the break-even, so that one batch mixes both modes.
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("B", [512, 2048, 4096])
def test_raw_fallback_of_multi_tile_shards(dtype, B):
    say(f"[gpu] RAW fallback multi-tile {dtype} B={B}")
    specs = [W.TensorSpec("a", 1, 30001), W.TensorSpec("b", 3, 25013), W.TensorSpec("c", 2, 65536 + 4097),
             W.TensorSpec("d", 1, 8192 * 3 + 15)]
    fracs = [0.6, 0.3, 0.18, 0.22] if dtype != torch.float32 else [0.6, 0.4, 0.3, 0.2]
    w0, w1 = [], []
    for i, (sp, f) in enumerate(zip(specs, fracs)):
        a = W.base_weights(sp, W.tensor_seed("rawfb", i), dtype)
        m = W.mask_uniform(sp.numel, f, W.tensor_seed("rawfb-m", i, B))
        w0.append(a)
        w1.append(W.perturb_exact(a, m, W.tensor_seed("rawfb-p", i, B)))
    case = Case([(sp.rows, sp.cols) for sp in specs], dtype, 1, B)
    res = case.run(w0, w1, compress=[1] * len(specs))
    assert res["status"] == 0 and res["ostatus"] == 0
    modes = [int(O.parse_header(case.codec.slot(i, 0).cpu().numpy())["mode"]) for i in range(len(specs))]
    assert modes[0] == O.MODE_RAW and O.MODE_RAW in modes


# (rows, cols, dtype, B, dense regions of 8192 values).  Shards of at most
# 2^21 values are encoded by one workgroup each; larger ones by the tiled split
# kernel (tiles of 8192 values for B <= 1024, 16384 for B = 2048, 32768 for
# B = 4096) and a finishing kernel: 1051 tiles go through the one that scans
# tile counts in windows of 1024, 129 and 65 tiles through the one with a
# workgroup per tile.  Dense regions (60%) overflow a tile's stash (a quarter
# of the tile), whose records are then derived again from the shard.
MANY_TILES = [
    (2101, 4096, torch.bfloat16, 512, (3, 1030, 1050)),
    (2101, 4096, torch.float16, 512, (3, 1030, 1050)),
    (2049, 1024, torch.bfloat16, 2048, (0, 1, 60, 256)),
    (2049, 1024, torch.float32, 4096, (4, 5, 6, 7, 200)),
    (2048, 1024, torch.bfloat16, 512, (0, 5, 255)),     # 2^21 values: one workgroup
    (2047, 1024, torch.float32, 512, (1, 254, 255)),
    (2048, 1024, torch.float16, 64, (0, 128, 255)),
]


@pytest.mark.parametrize("rows,cols,dtype,B,dense", MANY_TILES)
def test_many_tiles_and_stash_overflow(rows, cols, dtype, B, dense):
    """One shard at one rank: dense regions among 1% changes; the stream stays
    COMPRESSED."""
    T = 8192
    say(f"[gpu] many tiles {rows}x{cols} {dtype} B={B} dense {dense}")
    spec = W.TensorSpec("big", rows, cols)
    w0 = W.base_weights(spec, W.tensor_seed("many", rows, cols), dtype)
    mask = W.mask_uniform(rows * cols, 0.01, W.tensor_seed("many-m", rows, cols))
    dense_m = W.mask_uniform(rows * cols, 0.6, W.tensor_seed("many-d", rows, cols))
    for t in dense:
        lo, hi = t * T, min(rows * cols, (t + 1) * T)
        mask[lo:hi] |= dense_m[lo:hi]
    w1 = W.perturb_exact(w0, mask, W.tensor_seed("many-p", rows, cols))
    case = Case([(rows, cols)], dtype, 1, B)
    res = case.run([w0], [w1], compress=[1])
    assert res["status"] == 0 and res["ostatus"] == 0
    h = O.parse_header(case.codec.slot(0, 0).cpu().numpy())
    assert h["mode"] == O.MODE_COMPRESSED and h["n_changed"] > 0


# Decode searches of patch lists longer than 64 records, whose first round
# probes a window around the place an even spread predicts: shards of 256
# decode tiles (2048 x 1024 at one rank) whose changes are spread evenly, or
# sit far from where an even spread puts them, so that most keys fall outside
# their windows; lists from just above 64 records to above 2048.  (name,
# uniform rate, (first tile, last tile, rate) of denser regions in 8192-value
# tiles)
LONG_LISTS = [
    ("even-10pct", 0.10, ()),
    ("even-1.5pct", 0.015, ()),
    ("even-0.05pct", 0.0005, ()),
    ("first-tiles-only", 0.0, ((0, 1, 0.6),)),
    ("last-tile-only", 0.0, ((255, 255, 0.6),)),
    ("middle-cluster", 0.0005, ((100, 103, 0.6),)),
    ("every-eighth-tile", 0.0, tuple((t, t, 0.3) for t in range(3, 256, 8))),
    ("two-ends", 0.0, ((0, 0, 0.5), (250, 255, 0.2))),
    ("one-tile-short-list", 0.0, ((100, 100, 0.1),)),
    ("first-tile-short-list", 0.0, ((0, 0, 0.05),)),
    ("last-tile-short-list", 0.0, ((255, 255, 0.05),)),
    ("just-above-64", 0.0, ((10, 10, 0.01),)),
]


@pytest.mark.parametrize("name,frac,dense", LONG_LISTS)
def test_long_patch_lists(name, frac, dense):
    T = 8192
    rows, cols = 2048, 1024
    say(f"[gpu] long patch list {name}")
    spec = W.TensorSpec("long", rows, cols)
    w0 = W.base_weights(spec, W.tensor_seed("long", name), torch.bfloat16)
    mask = W.mask_uniform(rows * cols, frac, W.tensor_seed("long-m", name))
    for k, (t0, t1, f) in enumerate(dense):
        lo, hi = t0 * T, min(rows * cols, (t1 + 1) * T)
        mask[lo:hi] |= W.mask_uniform(hi - lo, f, W.tensor_seed("long-d", name, k))
    w1 = W.perturb_exact(w0, mask, W.tensor_seed("long-p", name))
    case = Case([(rows, cols)], torch.bfloat16, 1)
    res = case.run([w0], [w1], compress=[1])
    assert res["status"] == 0 and res["ostatus"] == 0
    h = O.parse_header(case.codec.slot(0, 0).cpu().numpy())
    assert h["mode"] == O.MODE_COMPRESSED and h["n_changed"] > 64


# Rows that some waves cover whole and others only in part: a wave whose 1024
# values of a 4096-value row are all in the shard moves them as contiguous
# 16-byte pieces swapped through LDS (encode loads of the values and fp32/fp16
# record stores; decode fp32/fp16 record loads and the rebuilt values of every
# type), the others lane by lane.  Shards end
# inside a row at a wave boundary, just past one, mid-wave and one value short.
WAVE_ROWS = [(1, 4096 + 1024), (1, 4096 + 1025), (1, 8192 + 3072 + 17), (1, 2 * 4096 - 1), (3, 7000),
             (1, 1024), (1, 1023), (5, 4096 + 2048 + 7)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("world", [1, 2])
def test_wave_rows_whole_and_partial(dtype, world):
    say(f"[gpu] whole and partial wave rows {dtype} W={world}")
    specs = [W.TensorSpec(f"w{i}", r * world, c) for i, (r, c) in enumerate(WAVE_ROWS)]
    cfg = W.PairConfig("wave-rows", dtype=dtype, frac=0.02)
    w0, w1 = _pairs(specs, cfg)
    for compress in ([1] * len(specs), [0] * len(specs)):
        res = Case([(s.rows, s.cols) for s in specs], dtype, world).run(w0, w1, compress=compress)
        assert res["status"] == 0 and res["ostatus"] == 0


def test_specials_and_all_bf16_patterns():
    """Every bf16 bit pattern (+-0, subnormals, Inf, all NaN payloads) survives."""
    say("[gpu] all 65536 bf16 patterns")
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).reshape(256, 256)
    rng = np.random.default_rng(5)
    perm = torch.from_numpy(rng.permutation(65536))
    w0 = [x.reshape(-1)[perm].reshape(256, 256).clone()]
    w1 = [x.clone()]
    for world in (1, 4, 16):
        res = Case([(256, 256)], torch.bfloat16, world).run(w0, w1, compress=[1])
        assert res["status"] == 0
    spec = [W.TensorSpec("r", 448, 256)]
    cfg = W.PairConfig("sp-test", frac=0.01, specials=1e-2)
    w0, w1 = _pairs(spec, cfg)
    assert Case([(448, 256)], torch.bfloat16, 16).run(w0, w1)["status"] == 0


def test_all_fp16_patterns_and_specials():
    """Every fp16 bit pattern (+-0, subnormals, Inf, all NaN payloads) survives,
    against a cache of other exponents, in shards of several sizes."""
    say("[gpu] all 65536 fp16 patterns")
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.float16).reshape(256, 256)
    rng = np.random.default_rng(6)
    perm = torch.from_numpy(rng.permutation(65536))
    w0 = [x.reshape(-1)[perm].reshape(256, 256).clone()]
    w1 = [x.clone()]
    for world in (1, 4, 16):
        res = Case([(256, 256)], torch.float16, world).run(w0, w1, compress=[1])
        assert res["status"] == 0
    spec = [W.TensorSpec("r", 448, 256)]
    cfg = W.PairConfig("sp16-test", dtype=torch.float16, frac=0.01, specials=1e-2)
    w0, w1 = _pairs(spec, cfg)
    assert Case([(448, 256)], torch.float16, 16).run(w0, w1)["status"] == 0


def _corrupt_case(frac=0.01):
    spec = [W.TensorSpec("k", 64, 3000)]
    a = W.base_weights(spec[0], 77, torch.bfloat16)
    m = W.mask_uniform(spec[0].numel, frac, 78)
    return spec, [a], [W.perturb_exact(a, m, 79)]


def test_decode_status_classes_match_oracle():
    spec, w0, w1 = _corrupt_case()
    rows, cols, world, B = 64, 3000, 4, 64
    n = 16 * cols
    ref = Case([(rows, cols)], torch.bfloat16, world, B)
    ref.run(w0, w1, compress=[1])
    s = ref.codec.slot(0, 1).cpu().numpy()
    h = O.parse_header(s)
    p = h["n_changed"]
    assert h["mode"] == O.MODE_COMPRESSED and p > 2
    nbm = O.bitmap_bytes(n, B)
    pb = 64 + n + nbm
    bm = s[64 + n:64 + n + nbm]
    j = int(np.nonzero(bm)[0][0])
    rec0, rec1 = bytes(s[pb:pb + 5]), bytes(s[pb + 5:pb + 10])
    edits = {
        "magic": [(0, 1, 0, b"X")],
        "version": [(0, 1, 4, b"\x07")],
        "dtype": [(0, 1, 6, b"\x02")],
        "mode": [(0, 1, 7, b"\x09")],
        "block": [(0, 1, 8, (128).to_bytes(4, "little"))],
        "n": [(0, 1, 16, (n + 1).to_bytes(8, "little"))],
        "offset": [(0, 1, 40, (1).to_bytes(8, "little"))],
        "rank": [(0, 1, 48, (2).to_bytes(4, "little"))],
        "world": [(0, 1, 52, (8).to_bytes(4, "little"))],
        "total_len": [(0, 1, 32, (int(h["total_len"]) + 5).to_bytes(8, "little"))],
        "n_changed": [(0, 1, 24, (p - 1).to_bytes(8, "little"))],
        "n_changed>n": [(0, 1, 24, (n + 1).to_bytes(8, "little"))],
        "index>=n": [(0, 1, pb + 5 * (p - 1), (n + 7).to_bytes(4, "little"))],
        "swap": [(0, 1, pb, rec1), (0, 1, pb + 5, rec0)],
        "duplicate": [(0, 1, pb + 5, rec0)],
        "bitmap-clear": [(0, 1, 64 + n + j, bytes([0]))],
        "bitmap-tail": [(0, 1, 64 + n + nbm - 1, bytes([int(bm[-1]) | 0x80]))],
    }
    assert O.n_blocks(n, B) % 8 != 0
    for name, e in edits.items():
        say(f"[gpu] corruption {name}")
        res = Case([(rows, cols)], torch.bfloat16, world, B).run(w0, w1, compress=[1], edits=e)
        g, o = res["status"], res["ostatus"]
        assert o != 0, name
        if o & O.ST_PATCH:          # bitmap bit unspecified alongside a patch error
            g &= ~O.ST_BITMAP
            o &= ~O.ST_BITMAP
        assert g == o, (name, g, o)


@pytest.mark.parametrize("frac", [0.01, 0.15])
def test_patch_record_order_errors_at_many_positions(frac):
    """Swapped and repeated patch records at many positions of a stream (first
    records of a lane, a wave, a pass of the record loop; the middle; the end)
    give the oracle's status.  At 1% a tile holds under one record per decode
    thread, at 15% several, so both record-loading paths are covered."""
    spec, w0, w1 = _corrupt_case(frac)
    rows, cols, world, B = 64, 3000, 4, 64
    n = 16 * cols
    ref = Case([(rows, cols)], torch.bfloat16, world, B)
    ref.run(w0, w1, compress=[1])
    s = ref.codec.slot(0, 1).cpu().numpy()
    h = O.parse_header(s)
    p = int(h["n_changed"])
    assert h["mode"] == O.MODE_COMPRESSED
    assert p > (2000 if frac > 0.1 else 300)
    pb = 64 + n + O.bitmap_bytes(n, B)
    rec = [bytes(s[pb + 5 * i:pb + 5 * i + 5]) for i in range(p)]
    pos = sorted({i for i in (0, 1, 3, 4, 63, 64, 255, 256, 1023, 1024, 1100, p // 2, p - 2) if i + 1 < p})
    for i in pos:
        for kind, e in (("swap", [(0, 1, pb + 5 * i, rec[i + 1]), (0, 1, pb + 5 * i + 5, rec[i])]),
                        ("repeat", [(0, 1, pb + 5 * i + 5, rec[i])])):
            res = Case([(rows, cols)], torch.bfloat16, world, B).run(w0, w1, compress=[1], edits=e)
            g, o = res["status"], res["ostatus"]
            assert o & O.ST_PATCH, (kind, i)
            assert g & ~O.ST_BITMAP == o & ~O.ST_BITMAP, (kind, i, g, o)


# Patch ranges of decode tiles (8192 values) whose element-patch lists are
# longer than 64 records: both tiles that share a boundary look for its place
# in the list, each on its own, probing a window around where an even spread
# puts it, so they must agree on it whatever the records hold.  (rows, cols,
# world, change rate): 490 records in six tiles, 121 in two, 1626 in two
# (about 813 a tile), 2446 in six.
RANGE_CASES = [(64, 3000, 4, 0.01), (16, 3000, 4, 0.01), (16, 1024, 1, 0.10), (64, 3000, 4, 0.05)]


@pytest.mark.parametrize("rows,cols,world,frac", RANGE_CASES)
def test_patch_ranges_at_tile_boundaries(rows, cols, world, frac):
    """Records swapped, repeated or moved across each tile boundary, and swapped
    at the places where the boundary's window begins and ends: the oracle's
    status, and where an edited list is still well formed, its values and
    cache."""
    T, B = 8192, 64
    say(f"[gpu] patch ranges at tile boundaries {rows}x{cols} W={world} f={frac}")
    spec = W.TensorSpec("ranges", rows, cols)
    a = W.base_weights(spec, W.tensor_seed("ranges", rows, cols), torch.bfloat16)
    m = W.mask_uniform(spec.numel, frac, W.tensor_seed("ranges-m", rows, cols))
    w0, w1 = [a], [W.perturb_exact(a, m, W.tensor_seed("ranges-p", rows, cols))]
    ref = Case([(rows, cols)], torch.bfloat16, world, B)
    ref.run(w0, w1, compress=[1])
    r = 0
    n = O.shard(rows, cols, world, r)[1]
    s = ref.codec.slot(0, r).cpu().numpy()
    h = O.parse_header(s)
    p = int(h["n_changed"])
    assert h["mode"] == O.MODE_COMPRESSED and p > 64 and n > T
    pb = 64 + n + O.bitmap_bytes(n, B)
    rec = [bytes(s[pb + 5 * i:pb + 5 * i + 5]) for i in range(p)]
    idx = np.array([int.from_bytes(x[:4], "little") for x in rec])
    edits = []
    for b in range(T, n, T):
        q = int(np.searchsorted(idx, b))  # first record of the tile that starts at b
        assert 0 < q < p
        for i in (q - 2, q - 1, q):
            if 0 <= i and i + 1 < p:
                edits.append((f"swap {i}", [(0, r, pb + 5 * i, rec[i + 1]), (0, r, pb + 5 * i + 5, rec[i])]))
                edits.append((f"repeat {i}", [(0, r, pb + 5 * i + 5, rec[i])]))
        if idx[q - 1] < b - 1:  # still ascending: the record moves to the tile before
            edits.append((f"move {q} to {b - 1}", [(0, r, pb + 5 * q, int(b - 1).to_bytes(4, "little"))]))
        if idx[q] > b:  # a record of the tile before moves to b
            edits.append((f"move {q - 1} to {b}", [(0, r, pb + 5 * (q - 1), int(b).to_bytes(4, "little"))]))
        for d in (16, 32, 48, 64, 65):  # near the ends of the probed windows (+-16 S records)
            for i in (q - d, q + d - 1):
                if 0 <= i and i + 1 < p:
                    edits.append((f"swap {i}", [(0, r, pb + 5 * i, rec[i + 1]), (0, r, pb + 5 * i + 5, rec[i])]))
    assert len(edits) > 10
    for name, e in edits:
        res = Case([(rows, cols)], torch.bfloat16, world, B).run(w0, w1, compress=[1], edits=e,
                                                                 valid_edits_decode=True)
        g, o = res["status"], res["ostatus"]
        if o & O.ST_PATCH:  # bitmap bit unspecified alongside a patch error
            g &= ~O.ST_BITMAP
            o &= ~O.ST_BITMAP
        assert g == o, (name, g, o)


def test_encode_is_deterministic():
    """Two encodes of the same inputs give identical bytes (no order dependence between workgroups)."""
    specs = W.olmoe_expert_specs()
    cfg = W.PairConfig("det", frac=0.01)
    w0, w1 = _pairs(specs, cfg)
    case = Case([(s.rows, s.cols) for s in specs], torch.bfloat16, 16)
    case.run(w0, w1)
    first = case.codec.streams.clone()
    for _ in range(3):
        case.run(w0, w1)
        assert torch.equal(first, case.codec.streams)


@pytest.mark.parametrize("polls", [1, 4])
def test_self_finishing_tiles_that_count_late_siblings(polls):
    """Tiles that finish their item themselves poll each sibling's change count
    a bounded number of times and otherwise count the sibling's changes from
    the shard and the cache.  With one or four polls most siblings are counted
    that way; every stream must still equal the oracle's, byte for byte
    (shards of 1 to 48 tiles, COMPRESSED and RAW fallback, three types)."""
    import lossless_weight_compression_amd as L
    say(f"[gpu] self-finishing tiles, {polls} polls")
    try:
        L.ciera_set_sync_polls(polls)
        for dtype in (torch.bfloat16, torch.float32, torch.float16):
            specs = [W.TensorSpec("a", 512, 768), W.TensorSpec("b", 96, 4096), W.TensorSpec("c", 7, 5)]
            w0, w1 = [], []
            for i, s in enumerate(specs):
                a = W.base_weights(s, W.tensor_seed("late", i), dtype)
                m = W.mask_uniform(s.numel, (0.01, 0.3, 0.2)[i], W.tensor_seed("late-m", i))
                w0.append(a)
                w1.append(W.perturb_exact(a, m, W.tensor_seed("late-p", i)))
            res = Case([(s.rows, s.cols) for s in specs], dtype, 2).run(w0, w1, compress=[1, 1, 1])
            assert res["status"] == 0 and res["ostatus"] == 0
    finally:
        L.ciera_set_sync_polls(0)
