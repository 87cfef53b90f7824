"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

Every mutation is a plausible slip -- a wrong shift, a dropped term, a flipped
bit order, an off-by-one that encode and decode share -- monkeypatched into the
oracle for the duration of one check."""
import numpy as np
import pytest

from oracle import ciera_oracle as O
from tests import test_oracle_brute_plan as TB
from tests import test_oracle_fields as TF
from tests import test_oracle_stream as TS
from tests import test_oracle_block as TBk
from tests import test_select as TSel
from tests import test_oracle_coded as TC

PINS = [
    TF.test_bf16_exponent_matches_frexp_exhaustive,
    TF.test_bf16_sign_mantissa_rebuilds_value_exhaustive,
    TF.test_known_values,
    TS.test_known_answer_bf16,
    TS.test_known_answer_fp32,
    TS.test_known_answer_fp16,
    TS.test_known_answer_fp16_partial_group,
    TF.test_fp16_fields_match_numpy_float16_exhaustive,
    TS.test_fp16_lengths_closed_form,
    TS.test_known_answer_fp32_raw_fallback,
    TS.test_known_answer_zero_change_and_plan_raw,
    TS.test_exhaustive_bf16_round_trip,
    TS.test_tie_is_raw,
    TS.test_payload_model_matches_pages,
    lambda: [TB.test_plan_decision_table(r) for r in TB.PLAN_TABLE],
    TB.test_corruption_classes,
    lambda: [TSel.test_select_table(r) for r in TSel.SELECT_TABLE],
    TSel.test_low_change_shards_rank_first,
    TBk.test_splitmix64_published_outputs,
    TBk.test_block_hash_position_length_and_avalanche,
    TBk.test_known_answer_block_stream,
    TBk.test_block_round_trip_all_bf16_patterns,
    TBk.test_block_decode_status_classes,
    TC.test_rans_worked_example,
    TC.test_rans_uniform_symbols_exact_length,
    TC.test_rans_table_symbols_entropy_bound,
    TC.test_interleaved_states_match_single_state_coding,
    TC.test_lane_counts,
    TC.test_chunk_symbols_worked_by_hand,
    TC.test_delta_classes,
    lambda: [TC.test_gap_buckets_follow_the_geometric_model(c, L) for c, L in ((41, 4096), (3, 100), (2000, 3000))],
    TC.test_gap_buckets_all_changed,
    TC.test_known_answer_stream_layout,
    TC.test_known_answer_padding_and_no_change,
    TC.test_dense_threshold,
    TC.test_round_trip_random_chunks_and_specials,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _wrong_exp_shift(u, dtype):
    u = np.asarray(u).astype(np.uint32)
    return ((u >> {O.BF16: 8, O.FP32: 23, O.FP16: 10}[dtype]) & (0x1F if dtype == O.FP16 else 0xFF)).astype(np.uint8)


def _sm_without_sign(u, dtype):
    u = np.asarray(u).astype(np.uint32)
    return u & {O.BF16: 0x7F, O.FP32: 0x7FFFFF, O.FP16: 0x3FF}[dtype]


def _fp16_exponent_eight_bits(orig):
    def ef(u, dtype):
        if dtype != O.FP16:
            return orig(u, dtype)
        return ((np.asarray(u).astype(np.uint32) >> 10) & 0xFF).astype(np.uint8)
    return ef


def _fp16_msb_first(orig_pack, orig_unpack):
    def pack(sm, dtype):
        if dtype != O.FP16:
            return orig_pack(sm, dtype)
        sm = np.asarray(sm).astype(np.uint32)
        bits = (sm[:, None] >> np.arange(11, dtype=np.uint32)[None, :]) & 1
        return np.packbits(bits.astype(np.uint8).reshape(-1), bitorder="big")

    def unpack(b, dtype, n=None):
        if dtype != O.FP16:
            return orig_unpack(b, dtype, n)
        bits = np.unpackbits(np.asarray(b, np.uint8), bitorder="big")[:11 * n].reshape(n, 11).astype(np.uint32)
        return (bits << np.arange(11, dtype=np.uint32)[None, :]).sum(axis=1).astype(np.uint32)
    return pack, unpack


def _fp16_two_bytes_per_value(orig):
    def smb(n, dtype):
        return 2 * n if dtype == O.FP16 else orig(n, dtype)
    return smb


def _comp_len_no_bitmap(n, p, dtype, B):
    base = O.HEADER_BYTES + O.sm_section_bytes(n, dtype)
    return base if p == 0 else base + O.PATCH_BYTES * p


def _comp_len_always_bitmap(n, p, dtype, B):
    return O.HEADER_BYTES + O.sm_section_bytes(n, dtype) + O.bitmap_bytes(n, B) + O.PATCH_BYTES * p


def _msb_first_encode(orig):
    def enc(*a, **k):
        s = orig(*a, **k)
        h = O.parse_header(s)
        if h["mode"] == O.MODE_COMPRESSED and h["n_changed"]:
            n = h["n"]
            off = 64 + O.sm_section_bytes(n, h["dtype"])
            nbm = O.bitmap_bytes(n, h["block_size"])
            bm = s[off:off + nbm]
            s = s.copy()
            s[off:off + nbm] = np.packbits(np.unpackbits(bm, bitorder="little"), bitorder="big")
        return s
    return enc


def _index_plus_one(orig_enc, orig_dec):
    def enc(*a, **k):
        s = orig_enc(*a, **k).copy()
        h = O.parse_header(s)
        if h["mode"] == O.MODE_COMPRESSED and h["n_changed"]:
            n, p = h["n"], h["n_changed"]
            pb = 64 + O.sm_section_bytes(n, h["dtype"]) + O.bitmap_bytes(n, h["block_size"])
            rec = s[pb:pb + 5 * p].reshape(p, 5)
            idx = rec[:, :4].copy().view("<u4").reshape(-1) + 1
            rec[:, :4] = idx.astype("<u4").view(np.uint8).reshape(p, 4)
        return s

    def dec(s, dtype, B, n, off, rank, world, cache_slice, coded=False):
        s = np.asarray(s, np.uint8).copy()
        try:
            h = O.parse_header(s)
        except ValueError:
            return orig_dec(s, dtype, B, n, off, rank, world, cache_slice, coded)
        if h["magic"] == O.MAGIC and h["mode"] == O.MODE_COMPRESSED and 0 < h["n_changed"] <= n:
            p = h["n_changed"]
            pb = 64 + O.sm_section_bytes(n, dtype) + O.bitmap_bytes(n, B)
            if pb + 5 * p <= s.size:
                rec = s[pb:pb + 5 * p].reshape(p, 5)
                idx = rec[:, :4].copy().view("<u4").reshape(-1) - 1
                rec[:, :4] = idx.astype("<u4").view(np.uint8).reshape(p, 4)
        return orig_dec(s, dtype, B, n, off, rank, world, cache_slice, coded)
    return enc, dec


def _decode_skips_patches(orig):
    def dec(s, dtype, B, n, off, rank, world, cache_slice, coded=False):
        x, ex, st = orig(s, dtype, B, n, off, rank, world, cache_slice, coded)
        if x is None or O.parse_header(np.asarray(s, np.uint8))["mode"] == O.MODE_RAW:
            return x, ex, st
        sm = O.sign_mantissa_field(x, dtype)
        return O.join_fields(sm, cache_slice, dtype), np.array(cache_slice), st
    return dec


def _plan_dec_without_world(rows, cols, dtype, B, world, ppm, cost=None):
    c = dict(O.DEFAULT_COST)
    _, n = O.shard(rows, cols, world, 0)
    raw = O.raw_len(n, dtype)
    p_hat = (ppm * n + 999_999) // 1_000_000
    comp = O.comp_len(n, p_hat, dtype, B)
    if comp >= raw:
        return dict(compress=0, expected_stream_bytes=raw, gain_ns=0)
    save = (raw - comp) * (world - 1) * 1000 // c["link_bytes_per_us"]
    dec = c["fixed_ns"] + (comp + 2 * n + n * O.elem_bytes(dtype)) * 1000 // c["hbm_bytes_per_us"]
    g = save - dec
    return dict(compress=int(g > 0), expected_stream_bytes=comp if g > 0 else raw, gain_ns=g)


def _check_raw_tie_compress(orig):
    def cl(n, p, dtype, B):
        return orig(n, p, dtype, B) - (1 if p else 0)
    return cl


def _select_variant(ascending=False, by_gain=False, skip_misfits=False, ties_reversed=False):
    """The selection with one plausible slip."""
    def sel(gains, cache, budget):
        from fractions import Fraction
        cand = [i for i in range(len(gains)) if gains[i] > 0]
        if ties_reversed:
            cand = cand[::-1]

        def key(i):
            if by_gain:
                return gains[i]
            return Fraction(gains[i], cache[i]) if cache[i] > 0 else float("inf")
        ranked = sorted(cand, key=key, reverse=not ascending)
        out, used = [0] * len(gains), 0
        for i in ranked:
            if used + cache[i] > budget:
                if skip_misfits:
                    continue
                break
            out[i], used = 1, used + cache[i]
        return out
    return sel


def _hash_without_position(b, seed):
    L = len(b)
    padded = bytes(b) + bytes(-L % 8)
    acc = 0
    for j in range(len(padded) // 8):
        w = int.from_bytes(padded[8 * j:8 * j + 8], "little")
        acc = (acc + O.mix64(w ^ seed)) & O.MASK64
    return O.mix64((acc + L) & O.MASK64)


def _mix64_wrong_shift(z):
    z = ((z ^ (z >> 31)) * 0xBF58476D1CE4E5B9) & O.MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & O.MASK64
    return z ^ (z >> 31)


def _block_len_unpadded(orig):
    def bl(n, c, dtype, B):
        full = orig(n, c, dtype, B)
        return full - (B - (n % B)) if c and n % B else full
    return bl


def _decode_blocks_ignores_payload(orig):
    def dec(s, pos, c, n, B, sm, ex, dtype):
        return O.join_fields(sm, ex, dtype), ex, 0
    return dec


def _rans_without_start(subs, lanes):
    x = [O.RANS_LOW] * lanes
    em = []
    for sub in reversed(subs):
        out = []
        for lane, start, f, k in sub:
            if x[lane] >= f << (32 - k):
                out.append((lane, x[lane] & 0xFFFF))
                x[lane] >>= 16
            x[lane] = ((x[lane] // f) << k) + x[lane] % f
        em.append([w for _, w in sorted(out)])
    return x, [w for sub in reversed(em) for w in sub]


def _rans_words_in_emission_order(orig):
    def enc(subs, lanes):
        x, w = orig(subs, lanes)
        return x, w[::-1]
    return enc


def _symbols_gap_without_minus_one(orig):
    def sym(offs, olds, news, length):
        subs, L = orig(offs, olds, news, length)
        gf = O.gap_bucket_freqs(len(offs), length)
        gc = [sum(gf[:i]) for i in range(13)]
        prev = 0  # gaps counted from the previous index itself
        out = []
        for t in range(len(subs) // 4):
            A, B = [], []
            for lane, *_ in subs[4 * t]:
                j = t * L + lane
                g = offs[j] - prev
                prev = offs[j]
                b = (g + 1).bit_length()
                A.append((lane, gc[b - 1], gf[b - 1], 12))
                if b > 1:
                    B.append((lane, (g + 1) - (1 << (b - 1)), 1, b - 1))
            out += [A, B, subs[4 * t + 2], subs[4 * t + 3]]
        return out, L
    return sym


def _symbols_escape_sends_step(orig):
    def sym(offs, olds, news, length):
        subs, L = orig(offs, olds, news, length)
        for t in range(len(subs) // 4):
            subs[4 * t + 3] = [(lane, (news[t * L + lane] - olds[t * L + lane]) & 0xFF, 1, 8)
                               for lane, *_ in subs[4 * t + 3]]
        return subs, L
    return sym


def _gap_freqs_unfixed(c, length):
    q = ((length - c) << 32) // length
    Q = [q]
    for _ in range(11):
        Q.append((Q[-1] * Q[-1]) >> 32)
    S = [1 << 32]
    for i in range(12):
        S.append((S[-1] * Q[i]) >> 32)
    share = [S[b - 1] - S[b] for b in range(1, 13)] + [S[12]]
    return [max(1, v >> 20) for v in share]


def _gap_freqs_shifted(orig):
    def gf(c, length):
        f = orig(c, length)
        return f[1:] + f[:1]
    return gf


def _delta_signs_swapped(orig_cls, orig_delta):
    def cls(old, new):
        k = orig_cls(old, new)
        return k ^ 1 if k < 14 else k

    def delta(k):
        return orig_delta(k ^ 1)
    return cls, delta


MUTATIONS = {
    "exponent shift off by one bit": lambda mp: mp.setattr(O, "exponent_field", _wrong_exp_shift),
    "sign bit dropped": lambda mp: mp.setattr(O, "sign_mantissa_field", _sm_without_sign),
    "bitmap length dropped": lambda mp: mp.setattr(O, "comp_len", _comp_len_no_bitmap),
    "bitmap kept when nothing changed": lambda mp: mp.setattr(O, "comp_len", _comp_len_always_bitmap),
    "bitmap most-significant bit first": lambda mp: mp.setattr(O, "encode", _msb_first_encode(O.encode)),
    "patch index off by one (shared)": lambda mp: (
        lambda ed: (mp.setattr(O, "encode", ed[0]), mp.setattr(O, "decode_stream", ed[1])))(
        _index_plus_one(O.encode, O.decode_stream)),
    "decode ignores patches": lambda mp: mp.setattr(O, "decode_stream", _decode_skips_patches(O.decode_stream)),
    "plan drops the W factor of decode": lambda mp: mp.setattr(O, "plan", _plan_dec_without_world),
    "tie resolved as compressed": lambda mp: mp.setattr(O, "comp_len", _check_raw_tie_compress(O.comp_len)),
    "fp16 exponent read as 8 bits": lambda mp: mp.setattr(O, "exponent_field", _fp16_exponent_eight_bits(O.exponent_field)),
    "fp16 bit stream most-significant bit first (shared)": lambda mp: (
        lambda pu: (mp.setattr(O, "pack_sm", pu[0]), mp.setattr(O, "unpack_sm", pu[1])))(
        _fp16_msb_first(O.pack_sm, O.unpack_sm)),
    "fp16 section sized 2 bytes per value": lambda mp: mp.setattr(O, "sm_section_bytes", _fp16_two_bytes_per_value(O.sm_section_bytes)),
    "selection ranked ascending": lambda mp: mp.setattr(O, "select", _select_variant(ascending=True)),
    "selection ranked by gain alone": lambda mp: mp.setattr(O, "select", _select_variant(by_gain=True)),
    "selection skips a misfit and goes on": lambda mp: mp.setattr(O, "select", _select_variant(skip_misfits=True)),
    "selection breaks ties against input order": lambda mp: mp.setattr(O, "select", _select_variant(ties_reversed=True)),
    "block hash without position key": lambda mp: mp.setattr(O, "block_hash64", _hash_without_position),
    "SplitMix64 mix with a wrong shift": lambda mp: mp.setattr(O, "mix64", _mix64_wrong_shift),
    "block payload last block unpadded": lambda mp: mp.setattr(O, "block_comp_len", _block_len_unpadded(O.block_comp_len)),
    "block decode ignores the payload": lambda mp: mp.setattr(O, "_decode_blocks", _decode_blocks_ignores_payload(O._decode_blocks)),
    "rANS symbol start dropped": lambda mp: mp.setattr(O, "rans_encode", _rans_without_start),
    "rANS words in emission order": lambda mp: mp.setattr(O, "rans_encode", _rans_words_in_emission_order(O.rans_encode)),
    "gap counted without the minus one": lambda mp: mp.setattr(O, "_chunk_symbols", _symbols_gap_without_minus_one(O._chunk_symbols)),
    "escape carries the step, not the exponent": lambda mp: mp.setattr(O, "_chunk_symbols", _symbols_escape_sends_step(O._chunk_symbols)),
    "coded padding dropped (shared)": lambda mp: mp.setattr(O, "pad4", lambda v: v),
    "gap table rounding not fixed": lambda mp: mp.setattr(O, "gap_bucket_freqs", _gap_freqs_unfixed),
    "gap table shifted one bucket": lambda mp: mp.setattr(O, "gap_bucket_freqs", _gap_freqs_shifted(O.gap_bucket_freqs)),
    "one state per 16 changes": lambda mp: mp.setattr(O, "rans_lanes", lambda c: min(64, (c + 15) // 16)),
    "dense from 1024 changes on": lambda mp: mp.setattr(O, "CODED_MAX_PATCHES", 1023),
    "exponent step signs swapped (shared)": lambda mp: (
        lambda cd: (mp.setattr(O, "delta_class", cd[0]), mp.setattr(O, "class_delta", cd[1])))(
        _delta_signs_swapped(O.delta_class, O.class_delta)),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    MUTATIONS[name](monkeypatch)
    assert _some_pin_fails(), f"no pin caught: {name}"


def test_unmutated_oracle_passes_all_pins():
    assert not _some_pin_fails()
