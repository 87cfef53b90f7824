"""Seeded synthetic weight tensors for the CIERA exponent-reuse codec.

Both sides of every parity check draw their inputs here: the CPU oracle
(under ``oracle/``) and the HIP path (the ``lossless_weight_compression_amd``
package).  This module only draws random numbers and perturbs them; it holds
none of the codec's own arithmetic (no exponent split, compare, bitmap, patch
list or stream layout).

What the pages fix about the workload (CIERA, arXiv 2609.04609v1):
  * the setting is sharded data parallelism over MoE expert weights, with the
    full tensor re-assembled by an Allgather every layer (abstract, section 1);
  * after warmup, well under 1% of exponents change between iterations, with
    post-warmup averages between 0.04% and 0.93% depending on learning rate and
    data (section 2.2, Figure 2); early iterations change far more;
  * OLMoE-1B-7B has 64 experts per layer (section 2).
The expert shapes, the change fractions {0, 0.1%, 1%, 10%}, the 4 KiB clustered
mode, fp32 master weights and the fine-grained 256-expert layer are the
synthetic stand-ins for trained checkpoints, which are not available here.

Recipe (all tensors are generated one at a time from their own seed):
  * base weights: fp32 N(0, 0.02^2); bf16 tensors are the round-to-nearest-even
    cast of those values;
  * additive perturbation (tiny case): W1 = W0 - 1e-3 * z * |W0|, z ~ N(0, 1),
    computed in fp32 from the stored W0 and cast back;
  * multiplicative perturbation: W1 = W0 * (1 + sigma * z), same casting;
  * exact masks: a chosen set of positions has the value doubled or halved
    (an exact operation for normal numbers, so its binary exponent moves by one)
    and every position has its low mantissa bits XOR-ed with fresh random bits,
    the way optimizer updates churn mantissas every step;
  * specials: each position independently becomes, with a given probability,
    one of {+0, -0, +subnormal, -subnormal, +Inf, -Inf, quiet NaN, signalling
    NaN}, NaNs with a random non-zero payload.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence, Tuple

import torch

BASE_STD = 0.02


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int

    @property
    def numel(self) -> int:
        return self.rows * self.cols


# ---------------------------------------------------------------- layer shapes

def tiny_specs() -> List[TensorSpec]:
    """One 256x512 matrix."""
    return [TensorSpec("tiny", 256, 512)]


def olmoe_expert_specs(expert: int = 0) -> List[TensorSpec]:
    """One OLMoE-1B-7B-shaped expert: gate and up 2048x1024, down 1024x2048."""
    return [TensorSpec(f"e{expert}.gate", 2048, 1024),
            TensorSpec(f"e{expert}.up", 2048, 1024),
            TensorSpec(f"e{expert}.down", 1024, 2048)]


def olmoe_layer_specs(n_experts: int = 64) -> List[TensorSpec]:
    """Full OLMoE-shaped MoE layer: 64 experts x 3 matrices, ~403M weights."""
    out: List[TensorSpec] = []
    for e in range(n_experts):
        out.extend(olmoe_expert_specs(e))
    return out


def fine_grained_layer_specs(n_experts: int = 256, d_model: int = 7168,
                             d_ffn: int = 2048, n_router: int = 256) -> List[TensorSpec]:
    """Fine-grained MoE layer: 256 experts x (7168x2048, 7168x2048, 2048x7168),
    a 7168x256 router and two RMSNorm vectors of 7168 (1-D: rows=7168, cols=1)."""
    out: List[TensorSpec] = []
    for e in range(n_experts):
        out.append(TensorSpec(f"e{e}.gate", d_model, d_ffn))
        out.append(TensorSpec(f"e{e}.up", d_model, d_ffn))
        out.append(TensorSpec(f"e{e}.down", d_ffn, d_model))
    out.append(TensorSpec("router", d_model, n_router))
    out.append(TensorSpec("norm.attn", d_model, 1))
    out.append(TensorSpec("norm.ffn", d_model, 1))
    return out


# ---------------------------------------------------------------------- seeds

def tensor_seed(*parts) -> int:
    """Deterministic 63-bit seed from any tuple of str/int parts."""
    h = hashlib.blake2b(repr(tuple(parts)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# ------------------------------------------------------------- base weights

def base_weights(spec: TensorSpec, seed: int, dtype: torch.dtype,
                 device="cpu", std: float = BASE_STD) -> torch.Tensor:
    """fp32 N(0, std^2) of shape (rows, cols), cast (RNE) to ``dtype``."""
    g = _gen(seed, device)
    w = torch.randn((spec.rows, spec.cols), generator=g, device=device,
                    dtype=torch.float32) * std
    return w.to(dtype)


def perturb_additive_abs(w0: torch.Tensor, seed: int, scale: float = 1e-3) -> torch.Tensor:
    """W1 = W0 - scale * z * |W0| in fp32, cast back to W0's dtype."""
    g = _gen(seed, w0.device)
    z = torch.randn(w0.shape, generator=g, device=w0.device, dtype=torch.float32)
    f = w0.float()
    return (f - scale * z * f.abs()).to(w0.dtype)


def perturb_multiplicative(w0: torch.Tensor, seed: int, sigma: float) -> torch.Tensor:
    """W1 = W0 * (1 + sigma * z) in fp32, cast back to W0's dtype."""
    g = _gen(seed, w0.device)
    z = torch.randn(w0.shape, generator=g, device=w0.device, dtype=torch.float32)
    return (w0.float() * (1.0 + sigma * z)).to(w0.dtype)


# sigma for which the multiplicative perturbation of bf16-cast N(0, 0.02^2)
# weights moves ~1% (resp. ~2%) of binary exponents (set by a bisection on
# a 2^22-element sample; the measured rate is reported wherever it is used).
SIGMA_1PCT = 0.0087
SIGMA_2PCT = 0.0174


# (mantissa bits, exponent bits, same-width integer type) of each float format
_LAYOUT = {torch.bfloat16: (7, 8, torch.int16), torch.float32: (23, 8, torch.int32),
           torch.float16: (10, 5, torch.int16)}


def elem_bytes(dtype: torch.dtype) -> int:
    return 4 if dtype == torch.float32 else 2


def _mantissa_mask(dtype: torch.dtype) -> int:
    return (1 << _LAYOUT[dtype][0]) - 1


def _int_view(w: torch.Tensor) -> torch.Tensor:
    return w.view(_LAYOUT[w.dtype][2])


def mask_uniform(numel: int, frac: float, seed: int, device="cpu") -> torch.Tensor:
    """Independent Bernoulli(frac) mask of length numel."""
    g = _gen(seed, device)
    if frac <= 0.0:
        return torch.zeros(numel, dtype=torch.bool, device=device)
    return torch.rand(numel, generator=g, device=device) < frac


def clustered_windows(specs: Sequence[TensorSpec], frac: float, elem_bytes: int,
                      seed: int, window_bytes: int = 4096) -> torch.Tensor:
    """Window ids for the clustered mode: the layer's tensors, in order, are one
    flat byte buffer cut into aligned ``window_bytes`` windows; K = round(frac *
    total_bytes / window_bytes) of them are drawn uniformly without
    replacement.  Every element inside a drawn window changes exponent."""
    total = sum(s.numel for s in specs) * elem_bytes
    n_win = (total + window_bytes - 1) // window_bytes
    k = int(round(frac * total / window_bytes))
    k = max(0, min(k, n_win))
    g = _gen(seed, "cpu")
    return torch.sort(torch.randperm(n_win, generator=g)[:k]).values


def mask_from_windows(windows: torch.Tensor, flat_elem_offset: int, numel: int,
                      elem_bytes: int, device="cpu", window_bytes: int = 4096) -> torch.Tensor:
    """Per-tensor mask from the layer-wide window ids (see clustered_windows)."""
    m = torch.zeros(numel, dtype=torch.bool, device=device)
    per = window_bytes // elem_bytes
    lo_b = flat_elem_offset * elem_bytes
    hi_b = (flat_elem_offset + numel) * elem_bytes
    sel = windows[(windows * window_bytes < hi_b) & ((windows + 1) * window_bytes > lo_b)]
    for w in sel.tolist():
        a = max(w * per - flat_elem_offset, 0)
        b = min((w + 1) * per - flat_elem_offset, numel)
        m[a:b] = True
    return m


def perturb_exact(w0: torch.Tensor, mask: torch.Tensor, seed: int) -> torch.Tensor:
    """Next iterate under an exact change mask.

    Masked positions are doubled or halved (random direction); this is exact
    for normal numbers away from the range limits, so their binary exponent
    moves by exactly one.  Every position then has its mantissa bits XOR-ed
    with random bits (which never touches the exponent)."""
    assert w0.dtype in _LAYOUT
    dev = w0.device
    g = _gen(seed, dev)
    flat = w0.reshape(-1)
    f = flat.float()
    up = torch.rand(flat.numel(), generator=g, device=dev) < 0.5
    scale = torch.where(up, torch.full_like(f, 2.0), torch.full_like(f, 0.5))
    f = torch.where(mask.reshape(-1), f * scale, f)
    w1 = f.to(w0.dtype)
    iv = _int_view(w1)
    mm = _mantissa_mask(w0.dtype)
    bits = torch.randint(0, mm + 1, (flat.numel(),), generator=g, device=dev,
                         dtype=torch.int64).to(iv.dtype)
    iv.bitwise_xor_(bits)
    return w1.reshape(w0.shape)


_SPECIALS = {
    # class -> (sign, exponent (0 or all ones), mantissa kind); kinds: 0 zero,
    # 1 random non-zero, 2 quiet NaN payload, 3 signalling NaN payload
    "pzero": (0, 0, 0), "nzero": (1, 0, 0),
    "psub": (0, 0, 1), "nsub": (1, 0, 1),
    "pinf": (0, 1, 0), "ninf": (1, 1, 0),
    "qnan": (None, 1, 2), "snan": (None, 1, 3),
}


def inject_specials(w: torch.Tensor, prob: float, seed: int) -> torch.Tensor:
    """Return a copy where each position, with probability ``prob``, is replaced
    by a value drawn uniformly from the eight special classes above.

    The bit patterns are built from the IEEE-754 / bfloat16 field positions:
    sign in the top bit, then the exponent (8 bits; 5 for fp16), then the
    mantissa (7 bits for bf16, 23 for fp32, 10 for fp16).  A quiet NaN has the
    top mantissa bit set; a signalling NaN has it clear and some other mantissa
    bit set."""
    dev = w.device
    g = _gen(seed, dev)
    out = w.clone().reshape(-1)
    n = out.numel()
    sel = torch.rand(n, generator=g, device=dev) < prob
    idx = sel.nonzero().reshape(-1)
    m = idx.numel()
    if m == 0:
        return out.reshape(w.shape)
    mbits, ebits, _ = _LAYOUT[w.dtype]
    emax = (1 << ebits) - 1
    cls = torch.randint(0, 8, (m,), generator=g, device=dev)
    rnd_sign = torch.randint(0, 2, (m,), generator=g, device=dev)
    rnd_mant = torch.randint(1, 1 << mbits, (m,), generator=g, device=dev)
    quiet_bit = 1 << (mbits - 1)
    sign = torch.zeros(m, dtype=torch.int64, device=dev)
    expo = torch.zeros(m, dtype=torch.int64, device=dev)
    mant = torch.zeros(m, dtype=torch.int64, device=dev)
    for c, (s, e, kind) in enumerate(_SPECIALS.values()):
        here = cls == c
        sign = torch.where(here, torch.full_like(sign, s) if s is not None else rnd_sign, sign)
        expo = torch.where(here, torch.full_like(expo, e * emax), expo)
        if kind == 1:
            mk = rnd_mant
        elif kind == 2:
            mk = rnd_mant | quiet_bit
        elif kind == 3:
            low = rnd_mant & (quiet_bit - 1)
            mk = torch.where(low == 0, torch.ones_like(low), low)
        else:
            mk = torch.zeros_like(mant)
        mant = torch.where(here, mk, mant)
    pattern = (sign << (mbits + ebits)) | (expo << mbits) | mant
    iv = _int_view(out)
    if w.dtype == torch.float32:
        pattern = torch.where(pattern >= 0x80000000, pattern - 0x100000000, pattern)
    else:
        pattern = torch.where(pattern >= 0x8000, pattern - 0x10000, pattern)
    iv[idx] = pattern.to(iv.dtype)
    return out.reshape(w.shape)


# ----------------------------------------------------------- config drivers

@dataclasses.dataclass
class PairConfig:
    """How to draw (W_prev, W_next) for one tensor of a layer."""
    tag: str                     # config name, part of every seed
    dtype: torch.dtype = torch.bfloat16
    kind: str = "exact"          # "additive", "multiplicative", "exact"
    sigma: float = 0.0           # multiplicative sigma
    frac: float = 0.0            # exact-mask change fraction
    clustered: bool = False      # exact masks: 4 KiB windows instead of Bernoulli
    specials: float = 0.0        # probability of a special value per position


def weight_pair(specs: Sequence[TensorSpec], i: int, cfg: PairConfig, device="cpu",
                windows: Optional[torch.Tensor] = None, iteration: int = 0,
                w_prev: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(W_prev, W_next) for tensor ``i`` of ``specs`` at ``iteration``.

    ``w_prev`` continues a chain of iterates; otherwise W_prev is the base
    weights (with specials injected if configured)."""
    s = specs[i]
    eb = elem_bytes(cfg.dtype)
    if w_prev is None:
        w_prev = base_weights(s, tensor_seed(cfg.tag, "base", i), cfg.dtype, device)
        if cfg.specials > 0:
            w_prev = inject_specials(w_prev, cfg.specials, tensor_seed(cfg.tag, "sp0", i))
    sd = tensor_seed(cfg.tag, "next", i, iteration)
    if cfg.kind == "additive":
        w_next = perturb_additive_abs(w_prev, sd)
    elif cfg.kind == "multiplicative":
        w_next = perturb_multiplicative(w_prev, sd, cfg.sigma)
    else:
        if cfg.clustered:
            assert windows is not None
            off = sum(x.numel for x in specs[:i])
            mask = mask_from_windows(windows, off, s.numel, eb, device)
        else:
            mask = mask_uniform(s.numel, cfg.frac, tensor_seed(cfg.tag, "mask", i, iteration), device)
        w_next = perturb_exact(w_prev, mask, sd)
    if cfg.specials > 0:
        w_next = inject_specials(w_next, cfg.specials, tensor_seed(cfg.tag, "sp", i, iteration + 1))
    return w_prev, w_next


def layer_windows(specs: Sequence[TensorSpec], cfg: PairConfig, iteration: int = 0) -> Optional[torch.Tensor]:
    if not cfg.clustered:
        return None
    eb = elem_bytes(cfg.dtype)
    return clustered_windows(specs, cfg.frac, eb, tensor_seed(cfg.tag, "win", iteration))


# Named configurations used by the tests and the benchmark.
def config(name: str, frac: float = 0.01, clustered: bool = False) -> Tuple[List[TensorSpec], PairConfig, int]:
    """(specs, pair config, world size) for a named workload."""
    if name == "tiny":
        return tiny_specs(), PairConfig("tiny", kind="additive"), 4
    if name == "tiny2pct":
        return tiny_specs(), PairConfig("tiny2pct", kind="multiplicative", sigma=SIGMA_2PCT), 4
    if name == "expert":
        return olmoe_expert_specs(), PairConfig("expert", kind="multiplicative", sigma=SIGMA_1PCT), 16
    if name == "layer":
        tag = f"layer-{frac}-{'c' if clustered else 'u'}"
        return olmoe_layer_specs(), PairConfig(tag, frac=frac, clustered=clustered), 16
    if name == "layer_fp32":
        tag = f"layer32-{frac}-{'c' if clustered else 'u'}"
        return olmoe_layer_specs(), PairConfig(tag, dtype=torch.float32, frac=frac,
                                               clustered=clustered), 16
    if name == "layer_fp16":
        tag = f"layer16-{frac}-{'c' if clustered else 'u'}"
        return olmoe_layer_specs(), PairConfig(tag, dtype=torch.float16, frac=frac,
                                               clustered=clustered), 16
    if name == "fine":
        return fine_grained_layer_specs(), PairConfig("fine", frac=frac, specials=1e-4), 16
    raise KeyError(name)
