"""Seeded random GPU parity cases against the oracle: batches of 1-4 tensors
with random shapes, world size, block size, element type, change rate and
pattern (uniform, clustered runs, special values), each tensor RAW, with
per-value patches or in the block-hash variant.  Everything is compared byte
for byte: streams, hash caches, rebuilt values, exponent caches, status."""
import numpy as np
import pytest
import torch

from gen import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_harness import say  # noqa: E402
from tests.test_gpu_block import run_block  # noqa: E402

DTYPES = [torch.bfloat16, torch.float32, torch.float16]


def _case(seed):
    rng = np.random.default_rng(seed)
    dtype = DTYPES[int(rng.integers(0, 3))]
    world = int(rng.choice([1, 2, 3, 4, 8, 16]))
    B = int(2 ** rng.integers(6, 13))
    shapes, w0, w1, variant = [], [], [], []
    for i in range(int(rng.integers(1, 5))):
        rows = int(rng.choice([1, world, int(rng.integers(1, 400))]))
        cols = int(rng.choice([1, 16, 333, int(rng.integers(1, 2500))]))
        spec = W.TensorSpec(f"r{i}", rows, cols)
        a = W.base_weights(spec, W.tensor_seed("rand", seed, i), dtype)
        frac = float(rng.choice([0.0, 1e-4, 1e-3, 1e-2, 0.1, 0.5]))
        if rng.random() < 0.3:  # clustered: whole runs of 256 values change
            m = torch.zeros(rows * cols, dtype=torch.bool)
            for s0 in range(0, rows * cols, 256):
                if rng.random() < max(frac, 0.02):
                    m[s0:s0 + 256] = True
        else:
            m = W.mask_uniform(rows * cols, frac, W.tensor_seed("rand-m", seed, i))
        b = W.perturb_exact(a, m, W.tensor_seed("rand-p", seed, i))
        if rng.random() < 0.3:
            a = W.inject_specials(a, 0.01, W.tensor_seed("rand-s0", seed, i))
            b = W.inject_specials(b, 0.01, W.tensor_seed("rand-s1", seed, i))
        shapes.append((rows, cols))
        w0.append(a)
        w1.append(b)
        variant.append(int(rng.choice([0, 1, 1, 2, 2])))
    return shapes, dtype, world, B, w0, w1, variant


@pytest.mark.parametrize("seed", range(40))
def test_random_batches(seed):
    shapes, dtype, world, B, w0, w1, variant = _case(seed)
    say(f"[gpu] random seed {seed}: {shapes} {dtype} W={world} B={B} variants {variant}")
    g, o = run_block(shapes, dtype, world, B, w0, w1, variant=variant)
    assert g == 0 and o == 0
