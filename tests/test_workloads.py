"""The seeded generator: determinism and the change rates each workload is meant to have."""
import numpy as np
import torch

from gen import workloads as W
from oracle import ciera_oracle as O


def _rate(a: torch.Tensor, b: torch.Tensor, dtype: int) -> float:
    ia = a.view(torch.int16 if dtype == O.BF16 else torch.int32).numpy().view(O.int_dtype(dtype))
    ib = b.view(torch.int16 if dtype == O.BF16 else torch.int32).numpy().view(O.int_dtype(dtype))
    return float(np.mean(O.exponent_field(ia, dtype) != O.exponent_field(ib, dtype)))


def test_deterministic():
    specs, cfg, _ = W.config("tiny")
    a0, a1 = W.weight_pair(specs, 0, cfg)
    b0, b1 = W.weight_pair(specs, 0, cfg)
    assert torch.equal(a0.view(torch.int16), b0.view(torch.int16))
    assert torch.equal(a1.view(torch.int16), b1.view(torch.int16))


def test_tiny_literal_formula_rate():
    """W1 = W0 - 1e-3 z |W0| moves far fewer than 2% of bf16 exponents: the
    relative step (~1e-3) is below bf16's resolution (2^-8), so most values
    round back.  The formula is kept literally; the 2% case is 'tiny2pct'."""
    specs, cfg, _ = W.config("tiny")
    r = _rate(*W.weight_pair(specs, 0, cfg), O.BF16)
    assert 1e-5 < r < 2e-3
    specs, cfg, _ = W.config("tiny2pct")
    r2 = _rate(*W.weight_pair(specs, 0, cfg), O.BF16)
    assert 0.015 < r2 < 0.025


def test_expert_multiplicative_near_one_percent():
    specs, cfg, _ = W.config("expert")
    rates = [_rate(*W.weight_pair(specs, i, cfg), O.BF16) for i in range(len(specs))]
    assert all(0.009 < r < 0.011 for r in rates), rates


def test_exact_uniform_rate_and_clustered_windows():
    specs = W.olmoe_expert_specs()
    cfg = W.PairConfig("t-exact", frac=0.01)
    w0, w1 = W.weight_pair(specs, 0, cfg)
    n = w0.numel()
    r = _rate(w0, w1, O.BF16)
    assert abs(r - 0.01) < 5 * np.sqrt(0.01 * 0.99 / n)
    # mantissas churn everywhere
    assert (w0.view(torch.int16) != w1.view(torch.int16)).float().mean() > 0.9
    cfg = W.PairConfig("t-clus", frac=0.01, clustered=True)
    win = W.layer_windows(specs, cfg)
    tot = sum(s.numel for s in specs) * 2
    assert win.numel() == round(0.01 * tot / 4096)
    changed = 0
    for i in range(3):
        a, b = W.weight_pair(specs, i, cfg, windows=win)
        ea = O.exponent_field(a.view(torch.int16).numpy().view(np.uint16), O.BF16)
        eb = O.exponent_field(b.view(torch.int16).numpy().view(np.uint16), O.BF16)
        d = np.nonzero(ea != eb)[0]
        changed += d.size
        # changes come in whole aligned 2048-element (4 KiB) windows
        if d.size:
            assert np.all(np.bincount(d // 2048) % 2048 == 0)
    assert changed == win.numel() * 2048


def test_specials_present():
    specs = W.tiny_specs()
    w = W.base_weights(specs[0], 1, torch.bfloat16)
    s = W.inject_specials(w, 0.05, 2).view(torch.int16).numpy().view(np.uint16)
    ex = O.exponent_field(s, O.BF16)
    sm = O.sign_mantissa_field(s, O.BF16)
    assert np.any((ex == 255) & ((sm & 0x7F) == 0))      # Inf
    assert np.any((ex == 255) & ((sm & 0x7F) != 0))      # NaN
    assert np.any((ex == 0) & ((sm & 0x7F) != 0))        # subnormal
    assert np.any((ex == 0) & (sm == 0x80))              # -0


def test_fp16_exact_rate_and_specials():
    """fp16 iterates: the exact mask moves the exponent of masked normal values
    by one (5-bit field), and the special classes land on the fp16 fields."""
    specs = W.olmoe_expert_specs()
    cfg = W.PairConfig("t-fp16", dtype=torch.float16, frac=0.01)
    w0, w1 = W.weight_pair(specs, 0, cfg)
    assert w0.dtype == torch.float16
    u0 = w0.reshape(-1).view(torch.int16).numpy().view(np.uint16)
    u1 = w1.reshape(-1).view(torch.int16).numpy().view(np.uint16)
    e0, e1 = O.exponent_field(u0, O.FP16).astype(int), O.exponent_field(u1, O.FP16).astype(int)
    normal = (e0 > 1) & (e0 < 30)
    moved = e0 != e1
    assert np.all(np.abs(e0 - e1)[moved & normal] == 1)
    n = u0.size
    assert abs(moved.mean() - 0.01) < 5 * np.sqrt(0.01 * 0.99 / n) + 0.004   # fp16 subnormal tail
    s = W.inject_specials(w0, 0.05, 3).reshape(-1).view(torch.int16).numpy().view(np.uint16)
    ex = O.exponent_field(s, O.FP16)
    m = O.sign_mantissa_field(s, O.FP16) & 0x3FF
    assert np.any((ex == 31) & (m == 0)) and np.any((ex == 31) & (m != 0))
    assert np.any((ex == 0) & (m != 0)) and np.any(s == 0x8000)
