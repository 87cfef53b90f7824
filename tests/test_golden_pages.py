"""The oracle against numbers the CIERA pages print (tests/golden/pages_block_model.txt).

Section 2.3's worked example of the uniform per-element model, its block-reuse
probability (1 - c)^B, and section 3.2's payload model with section 4.1's
block size."""
import math
import os

import numpy as np

from oracle import ciera_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_block_model.txt")


def _load():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (x.strip() for x in line.split("="))
            vals[k] = float(v)
    return vals


def test_worked_example_shard_unchanged():
    """(1 - 0.003)^(10^6) ~ e^-3000 (the pages round -3004.5 to -3000)."""
    g = _load()
    ln_p = g["uniform_n"] * math.log1p(-g["uniform_c"])
    assert abs(ln_p - g["log_pr_shard_unchanged"]) / abs(g["log_pr_shard_unchanged"]) < 0.01


def test_block_reuse_probability_in_oracle_bitmaps():
    """Blocks the oracle marks unchanged occur with probability (1 - c)^B at the
    pages' c = 0.003, for B = 64, 512 (the pages' default) and 1024."""
    g = _load()
    c = g["uniform_c"]
    rng = np.random.default_rng(2303)
    n = 1 << 21
    x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    exact = O.exponent_field(x, O.BF16)
    cache = np.where(rng.random(n) < c, exact ^ 1, exact).astype(np.uint8)
    for B in (64, int(g["block_size"]), 1024):
        s = O.encode(x, cache, O.BF16, B, True)
        nb = O.n_blocks(n, B)
        bm = np.unpackbits(s[64 + n:64 + n + O.bitmap_bytes(n, B)], bitorder="little")[:nb]
        reuse = 1.0 - bm.mean()
        want = (1 - c) ** B
        assert abs(reuse - want) < 5 * math.sqrt(want * (1 - want) / nb) + 1e-9, (B, reuse, want)


def test_payload_model_bitmap_bytes():
    """S_b = ceil(N/B), S_bm = ceil(S_b/8) at B = 512: the oracle's bitmap length."""
    B = int(_load()["block_size"])
    for N in (1, 511, 512, 513, 4096, 4097, 131072, 917504):
        sb = math.ceil(N / B)
        assert O.n_blocks(N, B) == sb and O.bitmap_bytes(N, B) == math.ceil(sb / 8)
