"""GPU parity of entropy-coded patches (stream mode 3: the changed exponents
range-ANS coded per 4096-value chunk, [CIERA 3.1; Algorithm 1 ANS-encode /
ANS-decode]) against the oracle, byte for byte: streams, rebuilt values,
exponent caches and decode status."""
import numpy as np
import pytest
import torch

from gen import workloads as W
from oracle import ciera_oracle as O

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from lossless_weight_compression_amd import _binding as B  # noqa: E402
from tests.gpu_harness import DT, say, to_np  # noqa: E402
from tests.test_gpu_block import run_block  # noqa: E402

_SHIFT = {torch.bfloat16: (7, 0xFF, torch.int16), torch.float16: (10, 0x1F, torch.int16),
          torch.float32: (23, 0xFF, torch.int32)}


def exponent_steps(w: torch.Tensor, mask: torch.Tensor, steps, seed: int) -> torch.Tensor:
    """w with the exponent field of the masked values moved by a step drawn
    from `steps` (modulo the field), every other bit kept."""
    sh, em, it = _SHIFT[w.dtype]
    g = torch.Generator().manual_seed(seed)
    u = w.reshape(-1).view(it).to(torch.int64) & ((1 << (8 * w.element_size())) - 1)
    st = torch.tensor(steps, dtype=torch.int64)[torch.randint(0, len(steps), (u.numel(),), generator=g)]
    e = (u >> sh) & em
    e2 = torch.where(mask.reshape(-1), (e + st) % (em + 1), e)
    u2 = (u & ~(em << sh)) | (e2 << sh)
    bits = 8 * w.element_size()
    u2 = torch.where(u2 >= 1 << (bits - 1), u2 - (1 << bits), u2)
    return u2.to(it).view(w.dtype).reshape(w.shape)


def _pair(rows, cols, dtype, frac, seed, steps=(1, -1), dense=()):
    spec = W.TensorSpec("c", rows, cols)
    w0 = W.base_weights(spec, W.tensor_seed("coded", seed), dtype)
    m = W.mask_uniform(rows * cols, frac, W.tensor_seed("coded-m", seed))
    for k, (lo, hi, f) in enumerate(dense):
        m[lo:hi] |= W.mask_uniform(hi - lo, f, W.tensor_seed("coded-d", seed, k))
    return w0, exponent_steps(w0, m, list(steps), W.tensor_seed("coded-p", seed))


CODED_EDGE = [
    # rows, cols, world, B, dtype, frac, exponent steps, dense ranges (value lo, hi, frac)
    (1, 1, 1, 512, torch.bfloat16, 1.0, (1,), ()),                      # RAW: not shorter
    (1, 1, 1, 512, torch.bfloat16, 0.0, (1,), ()),
    (17, 1, 16, 64, torch.bfloat16, 0.3, (1, -1), ()),
    (3, 5, 8, 512, torch.bfloat16, 0.2, (1, -1), ()),                   # ranks 3..7 hold no rows
    (10, 3, 4, 64, torch.bfloat16, 0.05, (1, -1, 9), ()),               # shard offsets not 16-aligned
    (10, 3, 4, 64, torch.float32, 0.05, (1, -1, 40), ()),
    (33, 7, 2, 128, torch.float16, 0.02, (1, -1, 5), ()),
    (1, 4097, 1, 512, torch.bfloat16, 0.001, (1, -1), ()),              # one value past a chunk
    (2, 8193, 1, 64, torch.bfloat16, 0.01, (1, -1, 2, -2, 100), ()),
    (64, 1000, 4, 1024, torch.bfloat16, 0.01, (1, -1), ()),             # tiles of 2 rows, wide blocks
    (64, 1000, 4, 2048, torch.float32, 0.003, (1, -1, 7, -7, 8), ()),   # tiles of 4 rows
    (96, 4096, 2, 4096, torch.bfloat16, 0.002, (1, -1), ()),            # tiles of 8 rows
    (96, 4096, 2, 4096, torch.float16, 0.0, (1,), ()),
    (1000, 1000, 16, 512, torch.bfloat16, 0.01, (1, -1), ()),
    (7168, 1, 16, 512, torch.bfloat16, 0.001, (1, -1), ()),
    (2048, 1024, 1, 512, torch.bfloat16, 0.01, (1, -1), ()),            # 256 tiles: one reduction
    (2101, 4096, 1, 512, torch.bfloat16, 0.01, (1, -1), ()),            # 1051 tiles: prefixes scanned
    (2049, 1024, 1, 2048, torch.float16, 0.002, (1, -1, 3),             # 129 tiles of 16384 values,
     ((0, 20000, 0.4), (2049 * 1024 - 5000, 2049 * 1024, 0.5))),        # dense runs at both ends
    (3001, 1024, 3, 512, torch.float32, 0.005, (1, -1), ()),            # 126 tiles per rank, 3 ranks
    (1200, 4096, 1, 512, torch.bfloat16, 0.3, (1, -1), ()),             # 601 tiles, RAW: not shorter
    (256, 1024, 1, 512, torch.bfloat16, 0.005, (1, -1),                 # dense chunks among coded ones
     ((4096, 8192, 0.6), (40000, 41000, 0.9), (262144 - 4096, 262144, 0.3))),
    (256, 1024, 1, 512, torch.bfloat16, 0.02, (1, -1, 3, -3, 50, 128), ()),  # many escapes
    (64, 4096, 1, 512, torch.bfloat16, 0.0, (1, -1),                    # exactly 1024 and 1025 changes
     ((0, 4096, 0.25), (4096, 8192, 0.26))),
    (64, 4096, 1, 512, torch.float16, 0.12, (1, -1, 4), ()),
    (64, 4096, 1, 512, torch.float32, 0.15, (1, -1), ()),
]


@pytest.mark.parametrize("rows,cols,world,Bk,dtype,frac,steps,dense", CODED_EDGE)
def test_coded_edge_shapes(rows, cols, world, Bk, dtype, frac, steps, dense):
    say(f"[gpu] coded {rows}x{cols} W={world} B={Bk} {dtype} f={frac} steps={steps} dense={dense}")
    w0, w1 = _pair(rows, cols, dtype, frac, (rows, cols, world, Bk, str(dtype), frac, steps), steps, dense)
    g, o = run_block([(rows, cols)], dtype, world, Bk, [w0], [w1], variant=[B.CODED])
    assert g == 0 and o == 0


def test_exact_1024_and_1025_changes_per_chunk():
    """Chunk 0 holds exactly 1024 changes (coded), chunk 1 exactly 1025 (dense)."""
    dtype = torch.bfloat16
    spec = W.TensorSpec("x", 2, 4096)
    w0 = W.base_weights(spec, W.tensor_seed("x1024"), dtype)
    rng = np.random.default_rng(3)
    m = torch.zeros(8192, dtype=torch.bool)
    m[torch.from_numpy(rng.choice(4096, 1024, replace=False))] = True
    m[4096 + torch.from_numpy(rng.choice(4096, 1025, replace=False))] = True
    w1 = exponent_steps(w0, m, [1, -1], 5)
    say("[gpu] coded 1024/1025")
    g, o = run_block([(2, 4096)], dtype, 1, 512, [w0], [w1], variant=[B.CODED])
    assert g == 0 and o == 0


# A last chunk shorter than 4096 values with more changes than its part of the
# output holds as 4-byte records (c > len * 2 / 4 for the two-byte types), yet
# coded shorter than dense: the prepass leaves it, and the merge decodes it
# itself.  (tail values, change rate in the tail)
MERGE_DECODED = [(100, 0.65), (37, 0.7), (1500, 0.6)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("tail,frac", MERGE_DECODED)
def test_coded_chunks_the_merge_decodes_itself(dtype, tail, frac):
    cols = 4096 + tail
    w0, w1 = _pair(1, cols, dtype, 0.0, ("merge-decoded", str(dtype), tail, frac), (1,), ((4096, cols, frac),))
    odt = DT[dtype]
    ex0 = O.exponent_field(to_np(w0), odt)[4096:]
    ex1 = O.exponent_field(to_np(w1), odt)[4096:]
    c = int(np.count_nonzero(ex0 != ex1))
    data = O.encode_chunk(ex1, ex0)
    assert c * 4 > tail * 2 and len(data) < O.pad4(tail), (c, len(data))  # the case meant
    say(f"[gpu] coded chunk of {tail} values, {c} changes, decoded by the merge, {dtype}")
    g, o = run_block([(1, cols)], dtype, 1, 512, [w0], [w1], variant=[B.CODED])
    assert g == 0 and o == 0


# Changes per 4096-value chunk of one shard, around the decoder's grouping of
# four consecutive chunks: quads whose chunks all hold at most 64 changes are
# decoded together, 16 lanes per chunk; any other quad one chunk at a time.
QUAD_COUNTS = [64, 1, 0, 64,      # packed, two chunks at the limit
               65, 2, 3, 0,       # one chunk past it
               0, 0, 0, 0,        # nothing to decode
               1024, 5, 64, 0,    # the most a coded chunk holds, beside small ones
               7, 0, 300]         # a quad cut short by the end of the shard


@pytest.mark.parametrize("dtype,world", [(torch.bfloat16, 1), (torch.bfloat16, 2), (torch.float32, 1),
                                         (torch.float16, 2)])
def test_chunk_quads_at_the_packing_limit(dtype, world):
    """Exact change counts per chunk at and past 64 in every quad position,
    empty quads, a full 1024-change chunk and a ragged last quad; escapes
    included.  Each rank's shard holds the same count pattern."""
    nch = len(QUAD_COUNTS)
    rows = nch * world
    spec = W.TensorSpec("q", rows, 4096)
    w0 = W.base_weights(spec, W.tensor_seed("quads", str(dtype), world), dtype)
    rng = np.random.default_rng(world * 7 + rows)
    m = torch.zeros(rows * 4096, dtype=torch.bool)
    for r in range(world):
        for k, c in enumerate(QUAD_COUNTS):
            base = (r * nch + k) * 4096
            m[base + torch.from_numpy(rng.choice(4096, c, replace=False))] = True
    w1 = exponent_steps(w0, m, [1, -1, 2, 100], W.tensor_seed("quads-p", str(dtype), world))
    say(f"[gpu] coded quads {dtype} W={world}")
    g, o = run_block([(rows, 4096)], dtype, world, 512, [w0], [w1], variant=[B.CODED])
    assert g == 0 and o == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("tail,tail_changes", [(1666, 1255), (1666, 600), (3000, 40), (2295, 1697)])
def test_partial_first_row_of_last_tile(dtype, tail, tail_changes):
    """A shard of six whole chunks and a partial one that opens the last
    encode tile (tiles of two rows), with few changes elsewhere: the partial
    chunk is dense by its count (more than 1024), or coded.  Its data length
    counts toward the stream's total length (a dense partial first row was
    once sized as a whole row)."""
    world, nch = 2, 6
    per = nch * 4096 + tail
    spec = W.TensorSpec("t", per * world, 1)
    w0 = W.base_weights(spec, W.tensor_seed("tail", str(dtype), tail, tail_changes), dtype)
    rng = np.random.default_rng(tail + tail_changes)
    m = torch.zeros(per * world, dtype=torch.bool)
    for r in range(world):
        for k in range(nch):
            m[r * per + k * 4096 + torch.from_numpy(rng.choice(4096, 40, replace=False))] = True
        m[r * per + nch * 4096 + torch.from_numpy(rng.choice(tail, tail_changes, replace=False))] = True
    w1 = exponent_steps(w0, m, [1, -1], W.tensor_seed("tail-p", str(dtype), tail))
    say(f"[gpu] coded partial first row {dtype} tail {tail} changes {tail_changes}")
    g, o = run_block([(per * world, 1)], dtype, world, 512, [w0], [w1], variant=[B.CODED])
    assert g == 0 and o == 0


# (B, row of the last tile that the partial chunk opens, dtype): tiles hold
# S = max(2, B / 512) rows; the shard is q * S + row whole chunks and a
# partial one, so the partial chunk is row `row` of its tile (rows 1..S-1)
PARTIAL_ROWS = ([(1024, 1, torch.bfloat16)] + [(2048, r, torch.bfloat16) for r in (1, 2, 3)]
                + [(4096, r, torch.bfloat16) for r in range(1, 8)]
                + [(2048, 3, torch.float32), (4096, 5, torch.float16), (4096, 7, torch.float32)])


@pytest.mark.parametrize("dense", [True, False])
@pytest.mark.parametrize("blk,row,dtype", PARTIAL_ROWS)
def test_partial_chunk_at_every_row_of_the_last_tile(blk, row, dtype, dense):
    """The partial chunk of a shard at each later row of the last encode tile,
    dense by its count (more than 1024 changes) or coded, among whole chunks
    with 40 changes each; the stream's total length and bytes must equal the
    oracle's.  (The length of a partial row was once folded to a whole row's
    when the partial chunk opened the tile.)"""
    S = max(2, blk // 512)
    nch = S + row
    tail, tail_changes = (2295, 1697) if dense else (3000, 40)
    world = 2
    per = nch * 4096 + tail
    spec = W.TensorSpec("t", per * world, 1)
    w0 = W.base_weights(spec, W.tensor_seed("rows", str(dtype), blk, row, dense), dtype)
    rng = np.random.default_rng(blk + 17 * row + dense)
    m = torch.zeros(per * world, dtype=torch.bool)
    for r in range(world):
        for k in range(nch):
            m[r * per + k * 4096 + torch.from_numpy(rng.choice(4096, 40, replace=False))] = True
        m[r * per + nch * 4096 + torch.from_numpy(rng.choice(tail, tail_changes, replace=False))] = True
    w1 = exponent_steps(w0, m, [1, -1], W.tensor_seed("rows-p", str(dtype), blk, row))
    say(f"[gpu] coded partial chunk at row {row} of {S}, B={blk} {dtype} dense={dense}")
    g, o = run_block([(per * world, 1)], dtype, world, blk, [w0], [w1], variant=[B.CODED])
    assert g == 0 and o == 0


@pytest.mark.parametrize("frac", [0.0, 0.001, 0.01, 0.1])
def test_coded_olmoe_expert_mixed_with_other_modes(frac):
    """One OLMoE expert, 16 ranks, in one batch: gate coded, up with element
    patches, down in the block-hash variant."""
    specs = W.olmoe_expert_specs()
    say(f"[gpu] coded expert f={frac}")
    w0, w1 = [], []
    for i, s in enumerate(specs):
        a = W.base_weights(s, W.tensor_seed("cx", i), torch.bfloat16)
        m = W.mask_uniform(s.numel, frac, W.tensor_seed("cx-m", i, frac))
        w0.append(a)
        w1.append(W.perturb_exact(a, m, W.tensor_seed("cx-p", i, frac)))
    g, o = run_block([(s.rows, s.cols) for s in specs], torch.bfloat16, 16, 512, w0, w1,
                     variant=[B.CODED, B.COMPRESSED, B.BLOCK])
    assert g == 0 and o == 0


def _mode3_case():
    rows, cols, world, Bk = 64, 3000, 4, 64
    w0, w1 = _pair(rows, cols, torch.bfloat16, 0.02, ("corrupt",), (1, -1, 9))
    return rows, cols, world, Bk, w0, w1


def test_coded_decode_status_classes_match_oracle():
    """Edited streams of rank 1 (48000 values, 12 chunks): header fields, table
    entries, states, words, dense data.  The bitmap verdict is unspecified
    alongside a length or patch error."""
    rows, cols, world, Bk, w0, w1 = _mode3_case()
    n = (rows // world) * cols
    ref = run_block([(rows, cols)], torch.bfloat16, world, Bk, [w0], [w1], variant=[B.CODED])
    assert ref == (0, 0)
    # the oracle's own stream for rank 1 gives the places to edit
    x1 = to_np(w1)
    cache0 = O.cache_update(to_np(w0), O.BF16)
    off, n1 = O.shard(rows, cols, world, 1)
    assert n1 == n
    s = O.encode_coded(x1[off:off + n], cache0[off:off + n], O.BF16, Bk, True, off, 1, world)
    h = O.parse_header(s)
    assert h["mode"] == O.MODE_CODED and h["n_changed"] > 100
    tpos = O.pad4(64 + n + O.bitmap_bytes(n, Bk))
    nch = O.n_chunks(n)
    dpos = tpos + 8 * nch
    tab = np.frombuffer(s[tpos:dpos].tobytes(), dtype="<u4")
    u32 = lambda v: int(v).to_bytes(4, "little")
    edits = {
        "mode 9": [(0, 1, 7, b"\x09")],
        "total short of the table": [(0, 1, 32, (dpos - 1).to_bytes(8, "little"))],
        "n_changed > n": [(0, 1, 24, (n + 1).to_bytes(8, "little"))],
        "count moved between chunks": [(0, 1, tpos + 8, u32(tab[2] + 1))],
        "last count": [(0, 1, tpos + 8 * (nch - 1), u32(tab[-2] + 1))],
        "bytes moved between chunks": [(0, 1, tpos + 4, u32(tab[1] + 4))],
        "bytes not a multiple of 4": [(0, 1, tpos + 4, u32(tab[1] + 2))],
        "table goes backwards": [(0, 1, tpos, u32(tab[2] + 1))],
        "bytes past the data": [(0, 1, tpos + 8 * 3 + 4, u32(tab[-1] + 400))],
        "state flipped": [(0, 1, dpos, bytes([s[dpos] ^ 1]))],
        "word flipped": [(0, 1, dpos + int(tab[1]) - 3, bytes([s[dpos + int(tab[1]) - 3] ^ 0x10]))],
        "bitmap bit": [(0, 1, 64 + n, bytes([s[64 + n] ^ 0x01]))],
        "bitmap tail": [(0, 1, 64 + n + O.bitmap_bytes(n, Bk) - 1,
                         bytes([int(s[64 + n + O.bitmap_bytes(n, Bk) - 1]) | 0x80]))],
        "coded longer than dense": [(0, 1, tpos + 4, u32(tab[1] + 4096)), (0, 1, tpos + 12, u32(tab[3] + 4096))],
    }
    assert O.n_blocks(n, Bk) % 8 != 0
    for name, e in edits.items():
        say(f"[gpu] coded corruption {name}")
        g, o = run_block([(rows, cols)], torch.bfloat16, world, Bk, [w0], [w1], edits=e, variant=[B.CODED])
        assert o != 0, name
        if o & (O.ST_LENGTH | O.ST_PATCH):
            g &= ~O.ST_BITMAP
            o &= ~O.ST_BITMAP
        assert g == o, (name, g, o)


DTYPES = [torch.bfloat16, torch.float32, torch.float16]


@pytest.mark.parametrize("seed", range(30))
def test_random_batches_with_coded(seed):
    """Batches of 1-4 tensors, random shapes, types, ranks, block sizes, change
    rates and exponent steps; each tensor coded, RAW, with element patches or
    in the block-hash variant."""
    rng = np.random.default_rng(1000 + seed)
    dtype = DTYPES[int(rng.integers(0, 3))]
    world = int(rng.choice([1, 2, 3, 4, 8, 16]))
    Bk = int(2 ** rng.integers(6, 13))
    shapes, w0, w1, variant = [], [], [], []
    for i in range(int(rng.integers(1, 5))):
        rows = int(rng.choice([1, world, int(rng.integers(1, 400))]))
        cols = int(rng.choice([1, 16, 333, int(rng.integers(1, 2500))]))
        frac = float(rng.choice([0.0, 1e-4, 1e-3, 1e-2, 0.05, 0.1, 0.5]))
        steps = [1, -1] if rng.random() < 0.6 else [1, -1, 2, -3, 7, -8, 60]
        dense = ()
        if rng.random() < 0.3 and rows * cols > 4096:
            lo = int(rng.integers(0, rows * cols - 4096))
            dense = ((lo, lo + 4096, float(rng.choice([0.3, 0.8]))),)
        a, b = _pair(rows, cols, dtype, frac, ("rc", seed, i), steps, dense)
        shapes.append((rows, cols))
        w0.append(a)
        w1.append(b)
        variant.append(int(rng.choice([3, 3, 3, 0, 1, 2])))
    say(f"[gpu] random coded seed {seed}: {shapes} {dtype} W={world} B={Bk} variants {variant}")
    g, o = run_block(shapes, dtype, world, Bk, w0, w1, variant=variant)
    assert g == 0 and o == 0


def test_receiver_without_coded_flag_rejects_mode_3():
    """A CODED stream reaching a decode whose tensor lacks CIERA_TENSOR_CODED is
    a mode mismatch (CIERA_ST_FIELD) and leaves the tensor untouched, as in the
    oracle."""
    from lossless_weight_compression_amd.layer import LayerCodec
    rows, cols, world = 64, 3000, 4
    w0, w1 = _pair(rows, cols, torch.bfloat16, 0.01, ("noflag",))
    say("[gpu] coded stream, receiver without the flag")
    A = LayerCodec([(rows, cols)], torch.bfloat16, world, 512, "cuda", 10_000, coded=[True])
    Bc = LayerCodec([(rows, cols)], torch.bfloat16, world, 512, "cuda", 10_000, coded=[False])
    d0, d1 = w0.to("cuda"), w1.to("cuda")
    A.seed_cache([d0])
    Bc.seed_cache([d0])
    for r in range(world):
        off, n = A.shard(0, r)
        A.encode(r, [d1.reshape(-1)[off:off + n].clone()], compress=[B.CODED])
    Bc.streams.copy_(A.streams)
    st = Bc.decode()
    torch.cuda.synchronize()
    x1, c0 = to_np(w1), O.cache_update(to_np(w0), O.BF16)
    slots = []
    for r in range(world):
        off, n = O.shard(rows, cols, world, r)
        s = O.encode_coded(x1[off:off + n], c0[off:off + n], O.BF16, 512, True, off, r, world)
        assert np.array_equal(A.slot(0, r)[:s.size].cpu().numpy(), s)
        slots.append(np.concatenate([s, np.zeros(16, np.uint8)]))
    _, o_cache, ost = O.decode(slots, rows, cols, O.BF16, 512, world, c0)
    assert ost == O.ST_FIELD and int(st.item()) == O.ST_FIELD
    assert np.array_equal(Bc.cache_view(0).cpu().numpy(), c0)
